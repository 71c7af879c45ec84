// libjscan: selective state-space scan (prefill and decode) for gfx950.
//
// The operation (see include/jscan.h) is the selective SSM recurrence of the
// "AI Engineering from Scratch" Jamba lesson, section "一页讲完 SSM": per
// channel d and state n, h = exp(delta*A[d][n]) * h + delta*B[n]*x, and
// y = (sum_n C[n]*h[n] + D[d]*x) * SiLU(z).  A is a real diagonal per
// (channel, state) as in Mamba-1 (same lesson, section "Mamba-3").
//
// Work decomposition on MI355X
// ----------------------------
// * Lanes map to channels: a wave covers 64 consecutive channels, so each
//   per-token load of x, delta and z is one coalesced 128-byte row segment.
// * The 16 states of a channel are split over K waves of one workgroup
//   (K = 1, 2, 4 or 8); wave g owns states [g*16/K, (g+1)*16/K).  The state
//   stays in VGPRs for the whole call.  Because a wave owns the same state
//   indices for all its lanes, the shared per-token rows B_t and C_t are
//   wave-uniform: they are read with scalar loads into SGPRs (bf16 pairs stay
//   packed and are widened by a scalar shift or mask) and fed to the VALU as
//   scalar operands, with no LDS traffic and no VGPRs.
// * With K > 1 the partial outputs sum_n C*h of the K waves are added through
//   LDS once per block of tokens, and each wave finishes (D skip, SiLU gate,
//   rounding, store) a 1/K share of the tokens.
// * When batch * d_inner is too small to give every SIMD two waves (one wave
//   per SIMD reaches only half the VALU issue rate on gfx950), the sequence
//   is cut into chunks scanned in parallel: a first kernel scans each chunk
//   from a zero state and keeps its end state S_c and its total delta; a
//   second combines the (decay, offset) pairs (P_c, S_c), P_c =
//   exp(A * sum delta), in order, seeded with h0, giving every chunk's
//   starting state; the main kernel then rescans each chunk from its true
//   starting state.
// * exp(delta*A) is computed as exp2(delta * (A*log2 e)), with A*log2 e
//   formed once per call in registers.
//
// All fp32 arithmetic; bf16 I/O is widened exactly on load and rounded to
// nearest-even on store.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <type_traits>

#include "jscan.h"

#include "common.h"
#include "host.h"

namespace jscan_detail {

// ------------------------------------------------- chunk-local end states
// One lane per channel, all 16 states.  Segment s (of the tokens before the
// last rescan chunk; every segment has seg_len tokens, a multiple of kTok) of
// sequence b: S[b][s][n][d] = state after the segment when it starts from
// zero, dsum[b][s][d] = sum of delta over the segment (accumulated in fp64).
// The workspace is state-major ([n][d]) so every access is a coalesced row.
// Waves per SIMD the main scan's register allocation is held to (the second
// __launch_bounds__ argument, amdgpu-waves-per-eu; 1 = no bound).  A SIMD
// lane has 512 VGPRs in granules of 8, so 4 waves allow 128.  The bf16
// trapezoidal scan needs 129 without a bound (3 waves); held to 4 waves it
// fits 121 without spilling VGPRs and runs its 64K prefill about 6% faster.
// Bounds on the other variants measured no gain and spill, so they have none.
template <class T, int K, bool CONV, bool SP, bool TR>
constexpr int scan_waves() { return sizeof(T) == 2 && K == 1 && TR ? 4 : 1; }

template <class T, bool CONV = false, bool SP = false, bool TR = false>
__global__ __launch_bounds__(256) void k_chunk_state(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, float* __restrict__ S, float* __restrict__ dsum,
    int64_t L, int64_t d_inner, int64_t seg_len, int n_segs, ProArgs pa) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t gbase = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (gbase >= d_inner) return;                       // whole wave past the end
  const int seg = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lo = (int)std::min<int64_t>(lane, d_inner - 1 - gbase);
  const int64_t d = gbase + lo;

  float a2[NSTATE], h[NSTATE];
  const float4* Ap = reinterpret_cast<const float4*>(A + d * NSTATE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float4 v = Ap[q];
    a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
    a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
  }
#pragma unroll
  for (int n = 0; n < NSTATE; ++n) h[n] = 0.0f;
  double dacc = 0.0;

  const int64_t t0 = (int64_t)seg * seg_len;
  const int nt = (int)seg_len;
  const T* xrow = x + (b * L + t0) * d_inner + gbase;
  const T* drow = delta + (b * L + t0) * d_inner + gbase;
  const T* brow = Bm + (b * L + t0) * NSTATE;
  const uint32_t lb = (uint32_t)lo * sizeof(T);      // lane byte offset within a row
  const uint32_t rowb = (uint32_t)(d_inner * sizeof(T));
  Prologue<CONV, SP> pro;
  pro.init(pa, d);
  pro.start(pa, pa.hist, x, b, L, d_inner, t0, d);
  // Trapezoidal form: the scan runs on the shifted state g (see trap_seed);
  // segment 0 starts from g_{-1} - h0 = w_0 B_prev, the combine adds h0.
  const T* lrow = TR && pa.lam ? static_cast<const T*>(pa.lam) + (b * L + t0) * d_inner + gbase : drow;
  const float lam_add = TR && !pa.lam ? 0.5f : 0.0f;      // a missing lam reads 0 through the empty resource
  if constexpr (TR) {
    if (t0 == 0) trap_seed(h, pa, pro, delta, b, L, d_inner, d, 0);
  }

  // Loads of token block bb (always kTok whole tokens: segments are multiples),
  // and with TR delta and lam of the token after the block (a segment never
  // ends the sequence, so that token exists).
  auto load_block = [&](int bb, T (&dd)[kTok], T (&xx)[kTok], T (&ll)[kTok], T& dn, T& ln) {
    const int64_t o = (int64_t)bb * d_inner;
    const auto rd = rsrc(drow + o), rx = rsrc(xrow + o);
    const auto rl = TR && pa.lam ? rsrc(lrow + o) : rsrc(drow, 0);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      buf_load(dd[j], rd, lb, j * rowb);
      buf_load(xx[j], rx, lb, j * rowb);
      if constexpr (TR) buf_load(ll[j], rl, lb, j * rowb);
    }
    if constexpr (TR) {
      buf_load(dn, rd, lb, kTok * rowb);
      buf_load(ln, rl, lb, kTok * rowb);
    }
  };
  Row<T, NSTATE> Bc, Bn;
  auto do_block = [&](int bb, const T (&dd)[kTok], const T (&xx)[kTok], const T (&ll)[kTok], const T& dn,
                      const T& ln) {
    float dtv[kTok + 1], lv[kTok + 1];             // TR: delta and lam of the block's tokens and the next
    if constexpr (TR) {
#pragma unroll
      for (int j = 0; j < kTok; ++j) { dtv[j] = pro.dt(widen(dd[j])); lv[j] = widen(ll[j]) + lam_add; }
      dtv[kTok] = pro.dt(widen(dn));
      lv[kTok] = widen(ln) + lam_add;
    }
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      Bn.load(brow + (int64_t)std::min(bb + j + 1, nt - 1) * NSTATE);
      const float dt = TR ? dtv[j] : pro.dt(widen(dd[j]));
      const float xv = pro.xin(widen(xx[j]));
      float dx = dt * xv;
      if constexpr (TR) dx = fmaf(dtv[j + 1] * (1.0f - lv[j + 1]), xv, dx * lv[j]);
      dacc += (double)dt;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dx * Bc[n]);
      Bc = Bn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Two register sets in turn: block i+1 is in flight while block i computes.
  T dA[kTok], xA[kTok], lA[kTok], dB[kTok], xB[kTok], lB[kTok], dnA, lnA, dnB, lnB;
  load_block(0, dA, xA, lA, dnA, lnA);
  Bc.load(brow);
  __builtin_amdgcn_s_waitcnt(0);
  for (int base = 0; base < nt; base += 2 * kTok) {
    load_block(std::min(base + kTok, nt - kTok), dB, xB, lB, dnB, lnB);
    do_block(base, dA, xA, lA, dnA, lnA);
    if (base + kTok >= nt) break;
    load_block(std::min(base + 2 * kTok, nt - kTok), dA, xA, lA, dnA, lnA);
    do_block(base + kTok, dB, xB, lB, dnB, lnB);
  }
  if (lo == lane) {
    const int64_t slot = b * n_segs + seg;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) S[(slot * NSTATE + n) * d_inner + d] = h[n];
    dsum[slot * d_inner + d] = (float)dacc;
  }
}

// ------------------------------------------------------------ carry combine
// One lane per (b, n, d), d fastest.  Folds the segments' (P, S) pairs in
// sequence order, h <- P * h + S with P = exp2(A' * dsum), seeded with h0,
// and records the state each rescan chunk starts from (every seg_per_chunk
// segments) in hstart[b][c][n][d].
//
// With a convolution prologue it also copies the conv history before the
// sequence into the workspace (hist_copy), so the rescan's first chunk never
// reads the caller's history buffer, which the last chunk may overwrite in
// place.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ A, const float* __restrict__ S,
                                                 const float* __restrict__ dsum, const float* __restrict__ h0,
                                                 float* __restrict__ hstart, int64_t d_inner, int n_chunks,
                                                 int seg_per_chunk, const float* __restrict__ hist,
                                                 float* __restrict__ hist_copy, int hist_rows,
                                                 int64_t* __restrict__ tag_out, Tag tag) {
  constexpr int G = 16;                // segments whose loads are in flight together
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (tag_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kTagWords)
    tag_out[threadIdx.x] = tag.w[threadIdx.x];
  const int64_t per_seq = d_inner * NSTATE;
  if (i >= per_seq) return;
  const int64_t n = i / d_inner;
  const int64_t d = i - n * d_inner;
  const int n_segs = (n_chunks - 1) * seg_per_chunk;
  if (hist_copy && n < hist_rows) {
    const int64_t o = (b * hist_rows + n) * d_inner + d;
    hist_copy[o] = hist ? hist[o] : 0.0f;
  }
  const float a2 = A[d * NSTATE + n] * kLog2e;
  const float* Sp = S + (b * n_segs) * per_seq + i;
  const float* Dp = dsum + (b * n_segs) * d_inner + d;
  float* Hp = hstart + (b * n_chunks) * per_seq + i;
  float h = h0 ? h0[(b * d_inner + d) * NSTATE + n] : 0.0f;
  Hp[0] = h;
  for (int s0 = 0; s0 < n_segs; s0 += G) {
    float sv[G], dv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int sg = std::min(s0 + k, n_segs - 1);
      sv[k] = Sp[(int64_t)sg * per_seq];
      dv[k] = Dp[(int64_t)sg * d_inner];
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int sg = s0 + k;
      if (sg < n_segs) {
        h = fmaf(fast_exp2(a2 * dv[k]), h, sv[k]);
        if ((sg + 1) % seg_per_chunk == 0) Hp[(int64_t)((sg + 1) / seg_per_chunk) * per_seq] = h;
      }
    }
  }
}

// ----------------------------------------------------------------- main scan
struct ScanArgs {
  const void* x; const void* delta; const float* A; const void* B; const void* C; const float* D;
  const void* z; const float* hinit;   // h0 (single chunk) or hstart (chunked), may be null
  void* y; float* hT;
  int64_t L, d_inner, chunk_len;
  int n_chunks;
  ProArgs pa;
};

// Grid: (ceil(d_inner / 64), chunks, batch); block: K waves.  Wave g of a
// block owns states [g*16/K, (g+1)*16/K) of the block's 64 channels for the
// block's chunk of tokens.
//
// Tokens go in blocks of kTok, the next block's loads issued before the
// current block is computed.  A chunk's last block may be partial: its
// missing tokens are loaded clamped onto the last token with delta = 0, so
// they leave the state bit-for-bit unchanged (exp2(0) = 1, input term
// 0 * x * B = 0 for finite x and B) and their output equals the last token's,
// which they store again to the same address.  Every block therefore runs the
// same branch-free code.
template <class T, int K, bool CONV = false, bool SP = false, bool TR = false>
__global__ __launch_bounds__(64 * K, (scan_waves<T, K, CONV, SP, TR>())) void k_scan(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dw, const T* __restrict__ z,
    const float* __restrict__ hinit, T* __restrict__ y, float* __restrict__ hT,
    int64_t L, int64_t d_inner, int64_t chunk_len, int n_chunks, ProArgs pa) {
  static_assert(K == 1 || !(CONV || SP || TR), "the input prologue and the trapezoidal form run with one wave "
                                              "per 64 channels");
  static_assert(!(CONV && TR), "the trapezoidal form takes no outer convolution");
  constexpr int S = NSTATE / K;
  constexpr int F = kTok / K;          // tokens of a block finished by each wave
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t gbase = (int64_t)blockIdx.x * 64;
  const int c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lo = (int)std::min<int64_t>(lane, d_inner - 1 - gbase);
  const int64_t d = gbase + lo;
  const int n0 = g * S;

  float a2[S], h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) a2[s] = A[d * NSTATE + n0 + s] * kLog2e;
  // Start state: hstart[b][c][n][d] (state-major) for chunked plans, else
  // h0[b][d][n] or zero.
  if (n_chunks > 1) {
    const float* hi = hinit + ((b * n_chunks + c) * NSTATE + n0) * d_inner + d;
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = hi[(int64_t)s * d_inner];
  } else {
    const float* hi = hinit ? hinit + (b * d_inner + d) * NSTATE + n0 : nullptr;
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = hi ? hi[s] : 0.0f;
  }
  const float Dd = Dw[d];

  const int64_t t0 = (int64_t)c * chunk_len;
  const int nt = (int)std::min<int64_t>(chunk_len, L - t0);   // >= 1 for every chunk
  const int64_t row0 = (b * L + t0) * d_inner + gbase;
  const T* xrow = x + row0;
  const T* drow = delta + row0;
  const T* zrow = z + row0;
  T* yrow = y + row0;
  const T* brow = Bm + (b * L + t0) * NSTATE + n0;
  const T* crow = Cm + (b * L + t0) * NSTATE + n0;

  __shared__ float red[K > 1 ? 2 : 1][K > 1 ? K : 1][kTok][64];

  const uint32_t lb = (uint32_t)lo * sizeof(T);      // lane byte offset within a row
  const uint32_t rowb = (uint32_t)(d_inner * sizeof(T));
  Prologue<CONV, SP> pro;
  pro.init(pa, d);
  pro.start(pa, pa.hist, x, b, L, d_inner, t0, d);
  // Trapezoidal form: the scan runs on the shifted state g (see trap_seed);
  // chunk 0 starts from h0 + w_0 B_prev, later chunks from the combine's g.
  const T* lrow = TR && pa.lam ? static_cast<const T*>(pa.lam) + row0 : drow;
  const float lam_add = TR && !pa.lam ? 0.5f : 0.0f;      // a missing lam reads 0 through the empty resource
  if constexpr (TR) {
    if (c == 0) trap_seed(h, pa, pro, delta, b, L, d_inner, d, n0);
  }

  // Loads of token block bb.  Rows past the chunk's end are clamped onto its
  // last token, and their delta is read through an empty resource (0).  With
  // TR also: delta and lam of the token after the block (0 past the
  // sequence's end), and for the block's C_t . B_t products lane l's pair of
  // states 2 (l & 7) + {0, 1} of token bb + (l >> 3), B and C.
  auto load_block = [&](int bb, T (&dd)[kTok], T (&xx)[kTok], T (&zz)[kTok], T (&ll)[kTok], T (&xff)[F],
                        T (&zff)[F], T& dn, T& ln, Pair<T>& pb, Pair<T>& pc) {
    const int64_t o = (int64_t)bb * d_inner;
    const auto rd = rsrc(drow + o), rx = rsrc(xrow + o), rz = rsrc(zrow + o), r0 = rsrc(drow, 0);
    const auto rl = TR && pa.lam ? rsrc(lrow + o) : r0;
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
      buf_load(dd[j], bb + j < nt ? rd : r0, lb, so);
      buf_load(xx[j], rx, lb, so);
      if constexpr (K == 1) buf_load(zz[j], rz, lb, so);
      if constexpr (TR) buf_load(ll[j], rl, lb, so);
    }
    if constexpr (TR) {
      const bool next = t0 + bb + kTok < L;
      buf_load(dn, next ? rd : r0, lb, kTok * rowb);
      buf_load(ln, next ? rl : r0, lb, kTok * rowb);
      const int jj = std::min(lane >> 3, nt - 1 - bb);
      const uint32_t vo = (uint32_t)(jj * NSTATE + 2 * (lane & 7)) * sizeof(T);
      pb.load(rsrc(brow + (int64_t)bb * NSTATE), vo);
      pc.load(rsrc(crow + (int64_t)bb * NSTATE), vo);
    }
    if constexpr (K > 1) {
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const uint32_t so = (uint32_t)(std::min(bb + i * K + g, nt - 1) - bb) * rowb;
        buf_load(xff[i], rx, lb, so); buf_load(zff[i], rz, lb, so);
      }
    }
  };

  // B of the next token is prefetched a token ahead; C is needed only after
  // the token's state updates, so it is loaded at the token's start.
  Row<T, S> Bc, Bn, Cv;
  int buf = 0;
  // y of token bb + j (padding tokens map onto the last token's address and
  // store the identical value again).
  // With a convolution, a padding token's input differs (its history has
  // shifted), so only real tokens store.
  auto finish = [&](__amdgpu_buffer_rsrc_t ry, int bb, int j, float acc, float xv, float zv) {
    const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
    if (!CONV || bb + j < nt) buf_store(to_io(fmaf(Dd, xv, acc) * silu(zv), T()), ry, lb, so);
  };
  auto do_block = [&](int bb, const T (&dd)[kTok], const T (&xx)[kTok], const T (&zz)[kTok],
                      const T (&ll)[kTok], const T (&xff)[F], const T (&zff)[F], const T& dn, const T& ln,
                      const Pair<T>& pb, const Pair<T>& pc) {
    const auto ry = rsrc(yrow + (int64_t)bb * d_inner);
    float part[kTok];
    // TR: delta and lam of the block's tokens and of the one after it (a
    // padding token's or a missing one's delta is 0), and C_t . B_t summed
    // over the 8 lanes of each token (lane 8 j holds token j's).
    float dtv[kTok + 1], lv[kTok + 1], cbl = 0.0f;
    if constexpr (TR) {
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        dtv[j] = bb + j < nt ? pro.dt(widen(dd[j])) : 0.0f;
        lv[j] = widen(ll[j]) + lam_add;
      }
      dtv[kTok] = t0 + bb + kTok < L ? pro.dt(widen(dn)) : 0.0f;
      lv[kTok] = widen(ln) + lam_add;
      cbl = pb.dot(pc);
      cbl += dpp_mov<0xB1>(cbl);        // lane ^ 1
      cbl += dpp_mov<0x4E>(cbl);        // lane ^ 2
      cbl += dpp_mov<0x141>(cbl);       // lane ^ 7 within 8 lanes
    }
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      Cv.load(crow + (int64_t)std::min(bb + j, nt - 1) * NSTATE);
      Bn.load(brow + (int64_t)std::min(bb + j + 1, nt - 1) * NSTATE);
      // A padding token's delta reads 0; softplus would turn that into a
      // positive step, so it is forced back to 0 (a wave-uniform select).
      const float dt = TR ? dtv[j] : SP ? (bb + j < nt ? pro.dt(widen(dd[j])) : 0.0f) : widen(dd[j]);
      const float xv = pro.xin(widen(xx[j]));
      float dx = dt * xv, wn = 0.0f;
      if constexpr (TR) {
        wn = dtv[j + 1] * (1.0f - lv[j + 1]) * xv;        // w_{t+1}
        dx = fmaf(dx, lv[j], wn);                          // dt lam x + w_{t+1}
      }
#pragma unroll
      for (int s = 0; s < S; ++s) h[s] = fmaf(fast_exp2(dt * a2[s]), h[s], dx * Bc[s]);
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) acc = fmaf(Cv[s], h[s], acc);
      if constexpr (TR) acc = fmaf(-wn, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cbl), 8 * j)), acc);
      if constexpr (K == 1) finish(ry, bb, j, acc, xv, widen(zz[j]));
      else part[j] = acc;
      Bc = Bn;
      // Keep each token's scalar B/C loads in its own token: hoisting them
      // across tokens would hold several rows in SGPRs at once and spill.
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (K > 1) {
      // Partial sums through LDS, double-buffered so one barrier per block
      // suffices: a wave overwrites buffer p only after the barrier of the
      // following block, which every wave reaches after its reads of p.
#pragma unroll
      for (int j = 0; j < kTok; ++j) red[buf][g][j][lane] = part[j];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < F; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < K; ++w) acc += red[buf][w][i * K + g][lane];
        finish(ry, bb, i * K + g, acc, widen(xff[i]), widen(zff[i]));
      }
      buf ^= 1;
    }
  };

  // Two register sets in turn: block i+1 is in flight while block i computes.
  T dA[kTok], xA[kTok], zA[kTok], lA[kTok], fxA[F], fzA[F], dnA, lnA;
  T dB[kTok], xB[kTok], zB[kTok], lB[kTok], fxB[F], fzB[F], dnB, lnB;
  Pair<T> pbA, pcA, pbB, pcB;
  load_block(0, dA, xA, zA, lA, fxA, fzA, dnA, lnA, pbA, pcA);
  Bc.load(brow);
  __builtin_amdgcn_s_waitcnt(0);
  // Prefetches past the chunk's end are clamped to its last block (valid rows,
  // values unused), so every row offset below stays non-negative.
  const int last = (nt - 1) / kTok * kTok;
  for (int base = 0; base < nt; base += 2 * kTok) {
    load_block(std::min(base + kTok, last), dB, xB, zB, lB, fxB, fzB, dnB, lnB, pbB, pcB);
    do_block(base, dA, xA, zA, lA, fxA, fzA, dnA, lnA, pbA, pcA);
    if (base + kTok >= nt) break;
    load_block(std::min(base + 2 * kTok, last), dA, xA, zA, lA, fxA, fzA, dnA, lnA, pbA, pcA);
    do_block(base + kTok, dB, xB, zB, lB, fxB, fzB, dnB, lnB, pbB, pcB);
  }
  if (hT && c == n_chunks - 1 && lo == lane) {
    float* ho = hT + (b * d_inner + d) * NSTATE + n0;
#pragma unroll
    for (int s = 0; s < S; ++s) ho[s] = h[s];
  }
  // Conv history after the sequence: its last width-1 raw x (read back from
  // x, or from the history before it when the sequence is shorter).  With
  // chunks > 1 every read here comes from x, so an in-place history is safe.
  if constexpr (CONV) {
    if (pa.hist_out && c == n_chunks - 1 && lo == lane) {
      for (int j = 0; j < pa.width - 1; ++j) {
        const float v = pro.before(pa, pa.hist, x, b, L, d_inner, L - (pa.width - 1) + j, d);
        pa.hist_out[(b * (pa.width - 1) + j) * d_inner + d] = v;
      }
    }
  }
}

// ------------------------------------------------------------ input RMSNorm
// RMSNorm before the scan, v / sqrt(mean v^2 + eps) * w, fp32 inside and the
// result rounded to the I/O dtype.  Rows of B and C: one thread per (token,
// tensor), all 16 entries; a null weight copies the row unchanged.
template <class T>
__global__ __launch_bounds__(256) void k_rms_rows(const T* __restrict__ B, const T* __restrict__ C,
                                                  const float* __restrict__ wB, const float* __restrict__ wC,
                                                  float eps, T* __restrict__ Bo, T* __restrict__ Co,
                                                  int64_t rows) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * rows; i += (int64_t)gridDim.x * 256) {
    const bool isC = i >= rows;
    const int64_t r = isC ? i - rows : i;
    const T* src = (isC ? C : B) + r * NSTATE;
    T* dst = (isC ? Co : Bo) + r * NSTATE;
    const float* w = isC ? wC : wB;
    float v[NSTATE], ss = 0.0f;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) {
      v[n] = widen(src[n]);
      ss = fmaf(v[n], v[n], ss);
    }
    const float inv = w ? 1.0f / sqrtf(ss * (1.0f / NSTATE) + eps) : 1.0f;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) store_io(dst + n, w ? v[n] * inv * w[n] : v[n]);
  }
}

// The time step over the d_inner channels of each token: one workgroup per
// token row (grid-stride over rows), the sum of squares reduced in-wave by
// shuffles and across the four waves through LDS.  Rows whose byte size is a
// multiple of 16 move through 16-byte vectors (8 bf16 or 4 fp32 per lane);
// rows of up to 256 x 4 vectors (8192 bf16 channels) stay in registers
// between the sum and the scaling, longer ones are read again.
template <class T>
__global__ __launch_bounds__(256) void k_rms_dt(const T* __restrict__ delta, const float* __restrict__ w, float eps,
                                                T* __restrict__ out, int64_t rows, int64_t d_inner) {
  constexpr int V = 16 / sizeof(T);                  // elements per 16-byte vector
  constexpr int R = 4;                               // vectors a lane can hold
  __shared__ float part[4];
  const bool vec = d_inner % V == 0;
  const bool held = vec && d_inner <= (int64_t)256 * V * R;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const T* src = delta + row * d_inner;
    T* dst = out + row * d_inner;
    float ss = 0.0f;
    uint4 buf[R];
    if (held) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t d = ((int64_t)r * 256 + threadIdx.x) * V;
        if (d < d_inner) {
          buf[r] = *reinterpret_cast<const uint4*>(src + d);
          const T* v = reinterpret_cast<const T*>(&buf[r]);
#pragma unroll
          for (int k = 0; k < V; ++k) ss = fmaf(widen(v[k]), widen(v[k]), ss);
        }
      }
    } else if (vec) {
      for (int64_t d = (int64_t)threadIdx.x * V; d < d_inner; d += 256 * V) {
        T v[V];
        *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(src + d);
#pragma unroll
        for (int k = 0; k < V; ++k) ss = fmaf(widen(v[k]), widen(v[k]), ss);
      }
    } else {
      for (int64_t d = threadIdx.x; d < d_inner; d += 256) {
        const float v = widen(src[d]);
        ss = fmaf(v, v, ss);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    __syncthreads();                                 // part[] of the previous row is consumed
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d_inner + eps);
    if (held) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t d = ((int64_t)r * 256 + threadIdx.x) * V;
        if (d < d_inner) {
          T v[V];
          *reinterpret_cast<uint4*>(v) = buf[r];
#pragma unroll
          for (int k = 0; k < V; ++k) v[k] = to_io(widen(v[k]) * inv * w[d + k], T());
          *reinterpret_cast<uint4*>(dst + d) = *reinterpret_cast<const uint4*>(v);
        }
      }
    } else if (vec) {
      for (int64_t d = (int64_t)threadIdx.x * V; d < d_inner; d += 256 * V) {
        T v[V];
        *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(src + d);
#pragma unroll
        for (int k = 0; k < V; ++k) v[k] = to_io(widen(v[k]) * inv * w[d + k], T());
        *reinterpret_cast<uint4*>(dst + d) = *reinterpret_cast<const uint4*>(v);
      }
    } else {
      for (int64_t d = threadIdx.x; d < d_inner; d += 256) store_io(dst + d, widen(src[d]) * inv * w[d]);
    }
  }
}

// Copy (or zero) the state for an empty sequence: hT = h0, or 0 when h0 is null.
__global__ __launch_bounds__(256) void k_copy_state(const float* __restrict__ src, float* __restrict__ dst,
                                                    int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// --------------------------------------------------------------- decode step
// Four lanes per (sequence, channel), four states each: the state row of a
// channel (64 bytes) is read and written as four float4s by adjacent lanes,
// so a wave moves 1 KiB of contiguous state per access.  The partial sums
// C.h of the four lanes are added with two xor shuffles inside the quad.
// With a convolution prologue the conv history of the channel
// (pa.hist[s][j][d], width-1 raw x) is read first and the shifted history,
// ending with this token's x, written by the quad's first lane (in place
// allowed).
template <class T, bool CONV = false, bool SP = false, bool TR = false>
__global__ __launch_bounds__(256) void k_step(float* __restrict__ state, const T* __restrict__ x,
                                              const T* __restrict__ delta, const float* __restrict__ A,
                                              const T* __restrict__ B, const T* __restrict__ C,
                                              const float* __restrict__ D, const T* __restrict__ z,
                                              T* __restrict__ y, int64_t n_seq, int64_t d_inner, ProArgs pa) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = n_seq * d_inner * 4;
  const bool active = gid < total;
  const int64_t g = active ? gid : total - 1;   // whole quads stay together: total % 4 == 0
  const int q = (int)(g & 3);
  const int64_t sd = g >> 2;
  const int64_t s = sd / d_inner;
  const int64_t d = sd - s * d_inner;

  float4 hv = reinterpret_cast<const float4*>(state)[g];
  const float4 av = reinterpret_cast<const float4*>(A)[d * 4 + q];
  Prologue<CONV, SP> pro;
  pro.init(pa, d);
  const float xraw = widen(x[sd]);
  float hist[3] = {0.f, 0.f, 0.f};              // oldest first: x[t-(width-1)] .. x[t-1]
  const int hw = pa.width - 1;                  // history length (0..3)
  if constexpr (CONV) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < hw && pa.hist) hist[j] = pa.hist[(s * hw + j) * d_inner + d];
    // x[t-1], x[t-2], x[t-3] out of the history, oldest first
    pro.h1 = hw == 3 ? hist[2] : hw == 2 ? hist[1] : hw == 1 ? hist[0] : 0.f;
    pro.h2 = hw == 3 ? hist[1] : hw == 2 ? hist[0] : 0.f;
    pro.h3 = hw == 3 ? hist[0] : 0.f;
  }
  const float xv = pro.xin(xraw);
  const float dt = pro.dt(widen(delta[sd]));
  const T* Bs = B + s * NSTATE + 4 * q;
  const T* Cs = C + s * NSTATE + 4 * q;
  float dx = dt * xv;
  if constexpr (TR) {
    // h = a (h + w B_prev) + v B with w = dt (1 - lam) x_prev, v = dt lam x
    const float lam = pa.lam ? widen(static_cast<const T*>(pa.lam)[sd]) : 0.5f;
    const float xp = pa.x_prev ? widen(static_cast<const T*>(pa.x_prev)[sd]) : 0.0f;
    const T* Bq = pa.B_prev ? static_cast<const T*>(pa.B_prev) + s * NSTATE + 4 * q : nullptr;
    const float wv = dt * (1.0f - lam) * xp;
    dx *= lam;
    if (Bq) {
      hv.x = fmaf(wv, widen(Bq[0]), hv.x);
      hv.y = fmaf(wv, widen(Bq[1]), hv.y);
      hv.z = fmaf(wv, widen(Bq[2]), hv.z);
      hv.w = fmaf(wv, widen(Bq[3]), hv.w);
    }
  }
  hv.x = fmaf(fast_exp2(dt * (av.x * kLog2e)), hv.x, dx * widen(Bs[0]));
  hv.y = fmaf(fast_exp2(dt * (av.y * kLog2e)), hv.y, dx * widen(Bs[1]));
  hv.z = fmaf(fast_exp2(dt * (av.z * kLog2e)), hv.z, dx * widen(Bs[2]));
  hv.w = fmaf(fast_exp2(dt * (av.w * kLog2e)), hv.w, dx * widen(Bs[3]));
  float part = widen(Cs[0]) * hv.x;
  part = fmaf(widen(Cs[1]), hv.y, part);
  part = fmaf(widen(Cs[2]), hv.z, part);
  part = fmaf(widen(Cs[3]), hv.w, part);
  part += __shfl_xor(part, 1, 4);
  part += __shfl_xor(part, 2, 4);
  if (active) {
    reinterpret_cast<float4*>(state)[g] = hv;
    if (q == 0) {
      store_io(y + sd, fmaf(D[d], xv, part) * silu(widen(z[sd])));
      if constexpr (CONV) {
        if (pa.hist_out) {
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (j < hw) pa.hist_out[(s * hw + j) * d_inner + d] = j + 1 < hw ? hist[j + 1] : xraw;
        }
      }
    }
  }
}

// ============================================================ host side
thread_local std::string t_last_error;
thread_local hipEvent_t t_ev_before = nullptr;
thread_local hipEvent_t t_ev_after = nullptr;
thread_local int t_force_K = 0;
thread_local int t_force_chunks = 0;

jscan_status fail(jscan_status s, const std::string& msg) {
  t_last_error = msg;
  return s;
}

jscan_status hip_fail(hipError_t e, const char* what) {
  t_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return JSCAN_ERR_HIP;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}


bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }


// Relative throughput of the scan loops with `waves` waves launched on the
// 1024 SIMDs, measured on MI355X with the one-wave-per-64-channels kernels
// (main scan at batch 1 and batch 8, d_inner 8192): one wave per SIMD issues
// at most every other cycle, a few more hide the load and exp latencies, and
// many more even out the tail across CUs.
double wave_efficiency(double waves) {
  static const double lw[] = {10, 11, 12, 13, 14, 15};
  static const double ef[] = {0.37, 0.53, 0.68, 0.91, 0.96, 1.0};
  const double l = std::log2(std::max(1.0, waves));
  if (l <= lw[0]) return ef[0] * waves / 1024.0;
  for (int i = 1; i < 6; ++i)
    if (l <= lw[i]) return ef[i - 1] + (ef[i] - ef[i - 1]) * (l - lw[i - 1]);
  return 1.0;
}

Plan make_plan(int64_t batch, int64_t L, int64_t d_inner, int K, int64_t C_target) {
  Plan p{K, 1, std::max<int64_t>(L, 1), 1, std::max<int64_t>(L, 1)};
  const int64_t groups = batch * ((d_inner + 63) / 64);
  if (L <= 0 || C_target <= 1 || groups <= 0) return p;
  // segments per chunk: about 32 chunk-local waves per SIMD (rounded down: the
  // combine's work grows with the segment count), >= 64 tokens each
  const int64_t want = (32 * 4 * kCUs) / (groups * (C_target - 1));
  int64_t F = std::max<int64_t>(1, std::min<int64_t>(want, (L / C_target) / kMinChunk));
  int64_t seg = (L + C_target * F - 1) / (C_target * F);
  seg = (seg + kTok - 1) / kTok * kTok;                    // whole token blocks
  int64_t chunk_len = seg * F;
  int64_t C = (L + chunk_len - 1) / chunk_len;
  if (C <= 1) return p;
  while ((C - 1) * F > 65535) { F = (F + 1) / 2; seg *= 2; chunk_len = seg * F; C = (L + chunk_len - 1) / chunk_len; }
  if (C <= 1) return p;
  return Plan{K, (int)C, chunk_len, (int)F, seg};
}

// Pick the plan.  Estimated time per channel-token: the rescan's VALU issue
// slots (about 150: 16 x (mul, exp at quarter rate, mul, fma, fma) plus the
// epilogue) over the efficiency its wave count reaches, plus the chunk-local
// pass (about 115 slots) on the (C-1)/C of the tokens that need a carry, over
// its own efficiency.  Measured on MI355X, splitting a channel's states over
// K > 1 waves never beat one wave per 64 channels with more chunks (the
// per-token work the K waves repeat and their barriers cost more than the
// extra chunk-local work), so the automatic plan keeps K = 1.
Plan choose_plan(int64_t batch, int64_t L, int64_t d_inner) {
  if (t_force_K > 0 && t_force_chunks > 0)
    return make_plan(batch, L, d_inner, t_force_K, std::min<int64_t>(t_force_chunks, std::max<int64_t>(L, 1)));
  const int64_t groups = batch * ((d_inner + 63) / 64);
  if (L <= 0 || groups <= 0) return make_plan(batch, L, d_inner, 1, 1);
  Plan best = make_plan(batch, L, d_inner, 1, 1);
  double best_cost = 1e300;
  for (int64_t C = 1; C <= 4096; C *= 2) {
    if (C > 1 && L / C < kMinChunk) break;
    const Plan p = make_plan(batch, L, d_inner, 1, C);
    double cost = 150.0 / wave_efficiency((double)groups * p.chunks);
    if (p.chunks > 1)
      cost += 115.0 * (double)(p.chunks - 1) / p.chunks / wave_efficiency((double)groups * p.segments());
    if (cost < best_cost * 0.999) { best = p; best_cost = cost; }
  }
  return best;
}

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }


WsLayout ws_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p) {
  WsLayout w{};
  if (p.chunks > 1) {
    const size_t segs = (size_t)p.segments();
    w.S = round_up((size_t)batch * segs * (size_t)d_inner * NSTATE * sizeof(float));
    w.dsum = round_up((size_t)batch * segs * (size_t)d_inner * sizeof(float));
    w.hstart = round_up((size_t)batch * (size_t)p.chunks * (size_t)d_inner * NSTATE * sizeof(float));
    w.hist = round_up((size_t)batch * 3 * (size_t)d_inner * sizeof(float));   // conv history copy
    w.tag = round_up(kTagWords * sizeof(int64_t));
  }
  w.total = w.tag + w.S + w.dsum + w.hstart + w.hist;
  return w;
}

Tag make_tag(int64_t batch, int64_t L, int64_t d_inner, const Plan& p, int variant) {
  return Tag{{kTagMagic, batch, L, d_inner, p.chunks, p.chunk_len, p.seg_per_chunk, variant}};
}

bool sizes_ok(int64_t batch, int64_t L, int64_t d_inner) {
  int64_t t;
  if (batch < 0 || L < 0 || d_inner < 0) return false;
  if (!mul_ok(batch, L, &t) || !mul_ok(t, d_inner, &t) || !mul_ok(t, 8, &t)) return false;
  if (!mul_ok(batch, d_inner, &t) || !mul_ok(t, NSTATE * 8, &t)) return false;
  if (!mul_ok(batch, L, &t) || !mul_ok(t, 32 * 8, &t)) return false;
  // 32-bit buffer offsets: a few rows of d_inner fp32 values, 64 chunks' tokens of B/C rows
  return L <= INT32_MAX && batch <= 65535 && d_inner <= (1 << 24);
}

template <class T, int K, bool CONV, bool SP, bool TR>
hipError_t launch_scan(const ScanArgs& a, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)((a.d_inner + 63) / 64), (unsigned)a.n_chunks, (unsigned)batch);
  hipLaunchKernelGGL((k_scan<T, K, CONV, SP, TR>), grid, dim3(64 * K), 0, st, static_cast<const T*>(a.x),
                     static_cast<const T*>(a.delta), a.A, static_cast<const T*>(a.B), static_cast<const T*>(a.C),
                     a.D, static_cast<const T*>(a.z), a.hinit,
                     static_cast<T*>(a.y), a.hT, a.L, a.d_inner, a.chunk_len, a.n_chunks, a.pa);
  return hipGetLastError();
}

template <class T, bool CONV, bool SP, bool TR>
hipError_t launch_scan_k(int K, const ScanArgs& a, int64_t batch, hipStream_t st) {
  if constexpr (CONV || SP || TR) {
    return launch_scan<T, 1, CONV, SP, TR>(a, batch, st);     // these run with K = 1
  } else {
    switch (K) {
      case 1: return launch_scan<T, 1, false, false, false>(a, batch, st);
      case 2: return launch_scan<T, 2, false, false, false>(a, batch, st);
      case 4: return launch_scan<T, 4, false, false, false>(a, batch, st);
      default: return launch_scan<T, 8, false, false, false>(a, batch, st);
    }
  }
}

template <class T, bool CONV, bool SP, bool TR>
jscan_status run_prefill(int64_t batch, int64_t L, int64_t d_inner, const void* x, const void* delta,
                         const float* A, const void* B, const void* C, const float* D, const void* z,
                         const float* h0, void* y, float* hT, char* ws, const Plan& p, const ProArgs& pa,
                         bool rms, hipStream_t st) {
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  float* S = reinterpret_cast<float*>(ws + w.off_S());
  float* dsum = reinterpret_cast<float*>(ws + w.off_dsum());
  float* hstart = reinterpret_cast<float*>(ws + w.off_hstart());
  float* hist_copy = reinterpret_cast<float*>(ws + w.off_hist());
  int64_t* tag_out = reinterpret_cast<int64_t*>(ws);
  const int variant = (CONV ? 1 : 0) | (SP ? 2 : 0) | (TR ? 4 : 0) | (rms ? 8 : 0);
  hipError_t e;

  ProArgs scan_pa = pa;
  if (p.chunks > 1) {
    const int segs = (int)p.segments();
    dim3 g1((unsigned)((d_inner + 255) / 256), (unsigned)segs, (unsigned)batch);
    hipLaunchKernelGGL((k_chunk_state<T, CONV, SP, TR>), g1, dim3(256), 0, st, static_cast<const T*>(x),
                       static_cast<const T*>(delta), A, static_cast<const T*>(B), S, dsum, L, d_inner, p.seg_len,
                       segs, pa);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "chunk-state launch");
    const int hist_rows = CONV ? pa.width - 1 : 0;
    dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
    hipLaunchKernelGGL(k_combine, g2, dim3(256), 0, st, A, S, dsum, h0, hstart, d_inner, p.chunks,
                       p.seg_per_chunk, pa.hist, hist_rows > 0 ? hist_copy : nullptr, hist_rows, tag_out,
                       make_tag(batch, L, d_inner, p, variant));
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "combine launch");
    if (hist_rows > 0) scan_pa.hist = hist_copy;
  }
  ScanArgs a{x, delta, A, B, C, D, z, p.chunks > 1 ? hstart : h0, y, hT, L, d_inner, p.chunk_len, p.chunks,
             scan_pa};
  hipEvent_t eb = t_ev_before, ea = t_ev_after;
  t_ev_before = t_ev_after = nullptr;
  if (eb && ea && (e = hipEventRecord(eb, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = launch_scan_k<T, CONV, SP, TR>(p.K, a, batch, st)) != hipSuccess) return hip_fail(e, "scan launch");
  if (eb && ea && (e = hipEventRecord(ea, st)) != hipSuccess) return hip_fail(e, "event record");
  return JSCAN_OK;
}

// Chunk starting states of a chunked plan (the chunk-local pass and the
// combine, without a prologue), for callers other than the prefill.
jscan_status forward_chunk_starts(jscan_io io, int64_t batch, int64_t L, int64_t d_inner, const void* x,
                                  const void* delta, const float* A, const void* B, const float* h0, char* ws,
                                  const Plan& p, hipStream_t st) {
  if (p.chunks <= 1) return JSCAN_OK;
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  float* S = reinterpret_cast<float*>(ws + w.off_S());
  float* dsum = reinterpret_cast<float*>(ws + w.off_dsum());
  float* hstart = reinterpret_cast<float*>(ws + w.off_hstart());
  const ProArgs none{nullptr, nullptr, nullptr, nullptr, nullptr, 1};
  const int segs = (int)p.segments();
  dim3 g1((unsigned)((d_inner + 255) / 256), (unsigned)segs, (unsigned)batch);
  if (io == JSCAN_IO_BF16)
    hipLaunchKernelGGL((k_chunk_state<uint16_t>), g1, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(delta), A, static_cast<const uint16_t*>(B), S, dsum, L,
                       d_inner, p.seg_len, segs, none);
  else
    hipLaunchKernelGGL((k_chunk_state<float>), g1, dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(delta), A, static_cast<const float*>(B), S, dsum, L, d_inner,
                       p.seg_len, segs, none);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "chunk-state launch");
  dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(k_combine, g2, dim3(256), 0, st, A, S, dsum, h0, hstart, d_inner, p.chunks, p.seg_per_chunk,
                     nullptr, nullptr, 0, nullptr, Tag{});
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "combine launch");
  return JSCAN_OK;
}

// Calls f(integral_constant<bool, CONV>, integral_constant<bool, SP>,
// integral_constant<bool, TR>) for the supported combinations (the
// trapezoidal form takes no convolution; callers reject that pair first).
template <class F>
auto with_flags(bool conv, bool sp, bool tr, F&& f) {
  using Y = std::true_type;
  using N = std::false_type;
  if (tr) return sp ? f(N{}, Y{}, Y{}) : f(N{}, N{}, Y{});
  if (conv && sp) return f(Y{}, Y{}, N{});
  if (conv) return f(Y{}, N{}, N{});
  if (sp) return f(N{}, Y{}, N{});
  return f(N{}, N{}, N{});
}

jscan_status check_common(int64_t d_state, jscan_io io) {
  if (io != JSCAN_IO_F32 && io != JSCAN_IO_BF16) return fail(JSCAN_ERR_UNSUPPORTED, "io must be JSCAN_IO_F32 or JSCAN_IO_BF16");
  if (d_state != NSTATE) return fail(JSCAN_ERR_UNSUPPORTED, "d_state must be 16");
  return JSCAN_OK;
}

// Every output against every input and every other output.  An output may be
// the very same buffer as one input (`same_ok`, e.g. an in-place state carry).
jscan_status check_ranges(const Range* in, int n_in, const Range* out, int n_out, const void* same_ok) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (!(same_ok && out[i].p == same_ok && in[j].p == same_ok && out[i].bytes == in[j].bytes) &&
          overlap(out[i], in[j]))
        return fail(JSCAN_ERR_ALIAS, std::string(out[i].name) + " overlaps " + in[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j]))
        return fail(JSCAN_ERR_ALIAS, std::string(out[i].name) + " overlaps " + out[j].name);
  }
  return JSCAN_OK;
}

template <class T, bool CONV, bool SP, bool TR>
jscan_status run_step(int64_t n_seq, int64_t d_inner, float* state, const void* x, const void* delta,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      void* y, const ProArgs& pa, hipStream_t st) {
  const int64_t total = n_seq * d_inner * 4;
  hipLaunchKernelGGL((k_step<T, CONV, SP, TR>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, state,
                     static_cast<const T*>(x), static_cast<const T*>(delta), A, static_cast<const T*>(B),
                     static_cast<const T*>(C), D, static_cast<const T*>(z), static_cast<T*>(y), n_seq,
                     d_inner, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "step launch");
  return JSCAN_OK;
}

bool has_rms(const jscan_prologue* pro) {
  return pro && (pro->rms_dt_weight || pro->rms_B_weight || pro->rms_C_weight);
}

// Validates the optional prologue and fills `pa`; appends its arrays to the
// input and output range lists for the alias check.  nseq = batch (prefill)
// or n_seq (step).
jscan_status check_prologue(const jscan_prologue* pro, int64_t nseq, int64_t d_inner, ProArgs* pa,
                            Range* in, int* n_in, Range* out, int* n_out) {
  *pa = ProArgs{nullptr, nullptr, nullptr, nullptr, nullptr, 1};
  if (!pro) return JSCAN_OK;
  if (has_rms(pro)) {
    if (!(pro->rms_eps >= 0.0f) || !std::isfinite(pro->rms_eps))
      return fail(JSCAN_ERR_UNSUPPORTED, "rms_eps must be finite and >= 0");
    const void* rp[] = {pro->rms_dt_weight, pro->rms_B_weight, pro->rms_C_weight};
    for (const void* p : rp)
      if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
    in[(*n_in)++] = Range{pro->rms_dt_weight, (size_t)d_inner * 4, "rms_dt_weight"};
    in[(*n_in)++] = Range{pro->rms_B_weight, NSTATE * 4, "rms_B_weight"};
    in[(*n_in)++] = Range{pro->rms_C_weight, NSTATE * 4, "rms_C_weight"};
  }
  if (pro->conv_weight) {
    if (pro->conv_width < 1 || pro->conv_width > 4)
      return fail(JSCAN_ERR_UNSUPPORTED, "conv_width must be 1..4");
    pa->conv_w = pro->conv_weight;
    pa->conv_b = pro->conv_bias;
    pa->hist = pro->conv_state_in;
    pa->hist_out = pro->conv_state_out;
    pa->width = pro->conv_width;
  } else if (pro->conv_bias || pro->conv_state_in || pro->conv_state_out) {
    return fail(JSCAN_ERR_NULL, "conv_bias / conv_state given without conv_weight");
  }
  if (pro->dt_softplus) pa->dt_bias = pro->dt_bias;
  const void* ptrs[] = {pro->conv_weight, pro->conv_bias, pro->conv_state_in, pro->conv_state_out,
                        pro->dt_bias};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const size_t hb = (size_t)nseq * (size_t)(pa->width - 1) * (size_t)d_inner * 4;
  in[(*n_in)++] = Range{pa->conv_w, (size_t)d_inner * pa->width * 4, "conv_weight"};
  in[(*n_in)++] = Range{pa->conv_b, (size_t)d_inner * 4, "conv_bias"};
  in[(*n_in)++] = Range{pa->hist, hb, "conv_state_in"};
  in[(*n_in)++] = Range{pro->dt_softplus ? pro->dt_bias : nullptr, (size_t)d_inner * 4, "dt_bias"};
  out[(*n_out)++] = Range{pa->hist_out, hb, "conv_state_out"};
  return JSCAN_OK;
}

// Normalises delta (over d_inner) and the B, C rows (over d_state) per token
// into stream-ordered scratch and points delta, B, C at the results; the
// caller frees *scratch after the scan.
jscan_status apply_rms(const jscan_prologue* pro, jscan_io io, int64_t nseq, int64_t L, int64_t d_inner,
                       const void** delta, const void** B, const void** C, void** scratch, hipStream_t st) {
  *scratch = nullptr;
  if (!has_rms(pro) || nseq == 0 || L == 0 || d_inner == 0) return JSCAN_OK;
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const int64_t rows = nseq * L;
  const size_t dbytes = pro->rms_dt_weight ? round_up((size_t)rows * (size_t)d_inner * es) : 0;
  const size_t rbytes = (pro->rms_B_weight || pro->rms_C_weight) ? round_up((size_t)rows * NSTATE * es) : 0;
  char* p = nullptr;
  hipError_t e;
  if ((e = hipMallocAsync(reinterpret_cast<void**>(&p), dbytes + 2 * rbytes, st)) != hipSuccess)
    return hip_fail(e, "hipMallocAsync(rmsnorm scratch)");
  *scratch = p;
  const unsigned grid_rows = (unsigned)std::min<int64_t>(rows, 1 << 20);
  if (pro->rms_dt_weight) {
    if (io == JSCAN_IO_BF16)
      hipLaunchKernelGGL((k_rms_dt<uint16_t>), dim3(grid_rows), dim3(256), 0, st,
                         static_cast<const uint16_t*>(*delta), pro->rms_dt_weight, pro->rms_eps,
                         reinterpret_cast<uint16_t*>(p), rows, d_inner);
    else
      hipLaunchKernelGGL((k_rms_dt<float>), dim3(grid_rows), dim3(256), 0, st, static_cast<const float*>(*delta),
                         pro->rms_dt_weight, pro->rms_eps, reinterpret_cast<float*>(p), rows, d_inner);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "rmsnorm launch");
    *delta = p;
  }
  if (rbytes) {
    char* bo = p + dbytes;
    char* co = bo + rbytes;
    const unsigned grid = (unsigned)std::min<int64_t>((2 * rows + 255) / 256, 1 << 20);
    if (io == JSCAN_IO_BF16)
      hipLaunchKernelGGL((k_rms_rows<uint16_t>), dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(*B),
                         static_cast<const uint16_t*>(*C), pro->rms_B_weight, pro->rms_C_weight, pro->rms_eps,
                         reinterpret_cast<uint16_t*>(bo), reinterpret_cast<uint16_t*>(co), rows);
    else
      hipLaunchKernelGGL((k_rms_rows<float>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(*B),
                         static_cast<const float*>(*C), pro->rms_B_weight, pro->rms_C_weight, pro->rms_eps,
                         reinterpret_cast<float*>(bo), reinterpret_cast<float*>(co), rows);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "rmsnorm launch");
    *B = bo;
    *C = co;
  }
  return JSCAN_OK;
}

// Validates the optional trapezoidal descriptor (I/O dtype arrays of element
// size es) and fills its fields of `pa`; appends its inputs to the range list.
jscan_status check_trap(const jscan_trap* tr, bool rms, int64_t nseq, int64_t L, int64_t d_inner, size_t es,
                        ProArgs* pa, Range* in, int* n_in) {
  if (!tr) return JSCAN_OK;
  if (pa->conv_w) return fail(JSCAN_ERR_UNSUPPORTED, "the trapezoidal form takes no convolution prologue");
  if (rms) return fail(JSCAN_ERR_UNSUPPORTED, "the trapezoidal form takes no RMSNorm prologue");
  const void* ptrs[] = {tr->lam, tr->x_prev, tr->B_prev};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  pa->lam = tr->lam;
  pa->x_prev = tr->x_prev;
  pa->B_prev = tr->B_prev;
  in[(*n_in)++] = Range{tr->lam, (size_t)nseq * (size_t)L * (size_t)d_inner * es, "lam"};
  in[(*n_in)++] = Range{tr->x_prev, (size_t)nseq * (size_t)d_inner * es, "x_prev"};
  in[(*n_in)++] = Range{tr->B_prev, (size_t)nseq * NSTATE * es, "B_prev"};
  return JSCAN_OK;
}

jscan_status prefill_impl(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                          const void* x, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* h0, void* y, float* hT,
                          const jscan_prologue* pro, const jscan_trap* trap, void* workspace,
                          size_t workspace_bytes, void* stream) {
  t_last_error.clear();
  jscan_status s = check_common(d_state, io);
  if (s != JSCAN_OK) return s;
  if (!sizes_ok(batch, L, d_inner)) return fail(JSCAN_ERR_SHAPE, "sizes must be >= 0 and fit 64-bit byte counts");
  const bool work = batch > 0 && L > 0 && d_inner > 0;
  if (work && (!x || !delta || !A || !B || !C || !D || !z || !y))
    return fail(JSCAN_ERR_NULL, "x, delta, A, B, C, D, z and y are required");
  const void* ptrs[] = {x, delta, A, B, C, D, z, h0, y, hT, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)batch * (size_t)L * (size_t)d_inner * es;
  const size_t rowb = (size_t)batch * (size_t)L * NSTATE * es;
  const size_t stb = (size_t)batch * (size_t)d_inner * NSTATE * 4;
  Plan plan = choose_plan(batch, L, d_inner);
  const size_t need = ws_layout(batch, L, d_inner, plan).total;
  Range in[20] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {B, rowb, "B"}, {C, rowb, "C"},
                  {A, (size_t)d_inner * NSTATE * 4, "A"}, {D, (size_t)d_inner * 4, "D"}, {h0, stb, "h0"}};
  Range out[4] = {{y, tok, "y"}, {hT, stb, "hT"}, {workspace, workspace ? need : 0, "workspace"}};
  int n_in = 8, n_out = 3;
  ProArgs pa;
  if ((s = check_prologue(pro, batch, d_inner, &pa, in, &n_in, out, &n_out)) != JSCAN_OK) return s;
  if ((s = check_trap(trap, has_rms(pro), batch, L, d_inner, es, &pa, in, &n_in)) != JSCAN_OK) return s;
  // An output may be the very same buffer as one input: hT == h0, or an
  // in-place conv history.
  for (int i = 0; i < n_out; ++i)
    for (int j = 0; j < n_in; ++j) {
      const bool same = out[i].p && out[i].p == in[j].p && out[i].bytes == in[j].bytes &&
                        ((out[i].p == (const void*)hT && in[j].p == (const void*)h0) ||
                         (out[i].p == (const void*)pa.hist_out && in[j].p == (const void*)pa.hist));
      if (!same && overlap(out[i], in[j]))
        return fail(JSCAN_ERR_ALIAS, std::string(out[i].name) + " overlaps " + in[j].name);
    }
  for (int i = 0; i < n_out; ++i)
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j]))
        return fail(JSCAN_ERR_ALIAS, std::string(out[i].name) + " overlaps " + out[j].name);
  if (workspace && workspace_bytes < need)
    return fail(JSCAN_ERR_WORKSPACE, "workspace smaller than jscan_prefill_workspace_size()");

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!work) {
    // Nothing to scan.  With L == 0 the final state and conv history are the initial ones.
    if (L == 0 && batch > 0 && d_inner > 0) {
      if (hT && hT != h0) {
        const int64_t n = batch * d_inner * NSTATE;
        hipLaunchKernelGGL(k_copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, h0, hT, n);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "state copy launch");
      }
      if (pa.hist_out && pa.hist_out != pa.hist && pa.width > 1) {
        const int64_t n = batch * (pa.width - 1) * d_inner;
        hipLaunchKernelGGL(k_copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pa.hist,
                           pa.hist_out, n);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "history copy launch");
      }
    }
    t_ev_before = t_ev_after = nullptr;
    return JSCAN_OK;
  }
  const bool conv = pa.conv_w != nullptr, sp = pro && pro->dt_softplus, tr = trap != nullptr;
  if (conv || sp || tr) plan.K = 1;                        // these run with one wave per group
  const void *dl = delta, *Bs = B, *Cs = C;
  void* rms_scratch = nullptr;
  if ((s = apply_rms(pro, io, batch, L, d_inner, &dl, &Bs, &Cs, &rms_scratch, st)) != JSCAN_OK) {
    if (rms_scratch) (void)hipFreeAsync(rms_scratch, st);
    return s;
  }
  char* ws = static_cast<char*>(workspace);
  bool owned = false;
  if (!ws && need > 0) {
    if ((e = hipMallocAsync(reinterpret_cast<void**>(&ws), need, st)) != hipSuccess) {
      if (rms_scratch) (void)hipFreeAsync(rms_scratch, st);
      return hip_fail(e, "hipMallocAsync(workspace)");
    }
    owned = true;
  }
  s = with_flags(conv, sp, tr, [&](auto cv, auto spv, auto trv) {
    constexpr bool CV = decltype(cv)::value, SPV = decltype(spv)::value, TRV = decltype(trv)::value;
    return io == JSCAN_IO_BF16
               ? run_prefill<uint16_t, CV, SPV, TRV>(batch, L, d_inner, x, dl, A, Bs, Cs, D, z, h0, y, hT, ws,
                                                     plan, pa, has_rms(pro), st)
               : run_prefill<float, CV, SPV, TRV>(batch, L, d_inner, x, dl, A, Bs, Cs, D, z, h0, y, hT, ws,
                                                  plan, pa, has_rms(pro), st);
  });
  if (owned) {
    e = hipFreeAsync(ws, st);
    if (s == JSCAN_OK && e != hipSuccess) s = hip_fail(e, "hipFreeAsync(workspace)");
  }
  if (rms_scratch) {
    e = hipFreeAsync(rms_scratch, st);
    if (s == JSCAN_OK && e != hipSuccess) s = hip_fail(e, "hipFreeAsync(rmsnorm scratch)");
  }
  return s;
}

jscan_status step_impl(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io, float* state,
                       const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, void* y, const jscan_prologue* pro,
                       const jscan_trap* trap, void* stream) {
  t_last_error.clear();
  jscan_status s = check_common(d_state, io);
  if (s != JSCAN_OK) return s;
  int64_t t;
  if (n_seq < 0 || d_inner < 0 || !mul_ok(n_seq, d_inner, &t) || !mul_ok(t, NSTATE * 16, &t) ||
      t / (NSTATE * 16) > ((int64_t)1 << 37))
    return fail(JSCAN_ERR_SHAPE, "sizes must be >= 0 and fit 64-bit byte counts");
  if (n_seq == 0 || d_inner == 0) {                       // nothing to do; the prologue is still checked
    Range in[12], out[1];
    int n_in = 0, n_out = 0;
    ProArgs pa;
    jscan_status s2 = check_prologue(pro, n_seq, d_inner, &pa, in, &n_in, out, &n_out);
    return s2 != JSCAN_OK ? s2 : check_trap(trap, has_rms(pro), n_seq, 1, d_inner, 4, &pa, in, &n_in);
  }
  if (!state || !x || !delta || !A || !B || !C || !D || !z || !y)
    return fail(JSCAN_ERR_NULL, "every pointer is required");
  const void* ptrs[] = {state, x, delta, A, B, C, D, z, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)n_seq * (size_t)d_inner * es;
  const size_t rowb = (size_t)n_seq * NSTATE * es;
  const size_t stb = (size_t)n_seq * (size_t)d_inner * NSTATE * 4;
  Range in[20] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {B, rowb, "B"}, {C, rowb, "C"},
                  {A, (size_t)d_inner * NSTATE * 4, "A"}, {D, (size_t)d_inner * 4, "D"}};
  Range out[3] = {{y, tok, "y"}, {state, stb, "state"}};
  int n_in = 7, n_out = 2;
  ProArgs pa;
  if ((s = check_prologue(pro, n_seq, d_inner, &pa, in, &n_in, out, &n_out)) != JSCAN_OK) return s;
  if ((s = check_trap(trap, has_rms(pro), n_seq, 1, d_inner, es, &pa, in, &n_in)) != JSCAN_OK) return s;
  if ((s = check_ranges(in, n_in, out, n_out, pa.hist_out && pa.hist_out == pa.hist ? pa.hist : nullptr)) !=
      JSCAN_OK)
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool conv = pa.conv_w != nullptr, sp = pro && pro->dt_softplus, tr = trap != nullptr;
  const void *dl = delta, *Bs = B, *Cs = C;
  void* rms_scratch = nullptr;
  if ((s = apply_rms(pro, io, n_seq, 1, d_inner, &dl, &Bs, &Cs, &rms_scratch, st)) != JSCAN_OK) {
    if (rms_scratch) (void)hipFreeAsync(rms_scratch, st);
    return s;
  }
  s = with_flags(conv, sp, tr, [&](auto cv, auto spv, auto trv) {
    constexpr bool CV = decltype(cv)::value, SPV = decltype(spv)::value, TRV = decltype(trv)::value;
    return io == JSCAN_IO_BF16
               ? run_step<uint16_t, CV, SPV, TRV>(n_seq, d_inner, state, x, dl, A, Bs, Cs, D, z, y, pa, st)
               : run_step<float, CV, SPV, TRV>(n_seq, d_inner, state, x, dl, A, Bs, Cs, D, z, y, pa, st);
  });
  if (rms_scratch) {
    const hipError_t e = hipFreeAsync(rms_scratch, st);
    if (s == JSCAN_OK && e != hipSuccess) s = hip_fail(e, "hipFreeAsync(rmsnorm scratch)");
  }
  return s;
}

}  // namespace jscan_detail

using namespace jscan_detail;

// ================================================================ C ABI
extern "C" {

const char* jscan_status_string(jscan_status s) {
  switch (s) {
    case JSCAN_OK: return "JSCAN_OK";
    case JSCAN_ERR_NULL: return "JSCAN_ERR_NULL";
    case JSCAN_ERR_SHAPE: return "JSCAN_ERR_SHAPE";
    case JSCAN_ERR_UNSUPPORTED: return "JSCAN_ERR_UNSUPPORTED";
    case JSCAN_ERR_ALIGN: return "JSCAN_ERR_ALIGN";
    case JSCAN_ERR_ALIAS: return "JSCAN_ERR_ALIAS";
    case JSCAN_ERR_WORKSPACE: return "JSCAN_ERR_WORKSPACE";
    case JSCAN_ERR_HIP: return "JSCAN_ERR_HIP";
  }
  return "JSCAN_UNKNOWN_STATUS";
}

const char* jscan_last_error(void) { return t_last_error.c_str(); }

void jscan_time_next_prefill(void* before, void* after) {
  t_ev_before = static_cast<hipEvent_t>(before);
  t_ev_after = static_cast<hipEvent_t>(after);
}

jscan_status jscan_set_plan_override(int waves_per_group, int chunks) {
  if (waves_per_group == 0 && chunks == 0) {
    t_force_K = t_force_chunks = 0;
    return JSCAN_OK;
  }
  if ((waves_per_group != 1 && waves_per_group != 2 && waves_per_group != 4 && waves_per_group != 8) ||
      chunks < 1 || chunks > 65535)
    return fail(JSCAN_ERR_UNSUPPORTED, "waves_per_group must be 1, 2, 4 or 8 and chunks in [1, 65535]");
  t_force_K = waves_per_group;
  t_force_chunks = chunks;
  return JSCAN_OK;
}

jscan_status jscan_prefill_plan(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                int* waves_per_group, int* chunks) {
  if (d_state != NSTATE) return fail(JSCAN_ERR_UNSUPPORTED, "d_state must be 16");
  if (!sizes_ok(batch, L, d_inner)) return fail(JSCAN_ERR_SHAPE, "invalid sizes");
  const Plan p = choose_plan(batch, L, d_inner);
  if (waves_per_group) *waves_per_group = p.K;
  if (chunks) *chunks = p.chunks;
  return JSCAN_OK;
}

size_t jscan_prefill_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                    jscan_io io) {
  if (d_state != NSTATE || (io != JSCAN_IO_F32 && io != JSCAN_IO_BF16)) return 0;
  if (!sizes_ok(batch, L, d_inner)) return 0;
  return ws_layout(batch, L, d_inner, choose_plan(batch, L, d_inner)).total;
}

jscan_status jscan_prefill(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                           const void* x, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* h0,
                           void* y, float* hT, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return prefill_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, y, hT, nullptr, nullptr,
                      workspace, workspace_bytes, stream);
}

jscan_status jscan_prefill_fused(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                 const void* x, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* h0,
                                 void* y, float* hT, const jscan_prologue* prologue, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return prefill_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, y, hT, prologue, nullptr,
                      workspace, workspace_bytes, stream);
}

jscan_status jscan_step_batch(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                              float* state, const void* x, const void* delta, const float* A,
                              const void* B, const void* C, const float* D, const void* z,
                              void* y, void* stream) {
  return step_impl(n_seq, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, nullptr, nullptr, stream);
}

jscan_status jscan_step_batch_fused(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                    float* state, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    void* y, const jscan_prologue* prologue, void* stream) {
  return step_impl(n_seq, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, prologue, nullptr, stream);
}

jscan_status jscan_prefill_trap(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                const void* x, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* h0, void* y, float* hT,
                                const jscan_trap* trap, const jscan_prologue* prologue, void* workspace,
                                size_t workspace_bytes, void* stream) {
  static const jscan_trap plain{nullptr, nullptr, nullptr};
  return prefill_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, y, hT, prologue,
                      trap ? trap : &plain, workspace, workspace_bytes, stream);
}

jscan_status jscan_step_batch_trap(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io, float* state,
                                   const void* x, const void* delta, const float* A, const void* B,
                                   const void* C, const float* D, const void* z, void* y,
                                   const jscan_trap* trap, const jscan_prologue* prologue, void* stream) {
  static const jscan_trap plain{nullptr, nullptr, nullptr};
  return step_impl(n_seq, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, prologue,
                   trap ? trap : &plain, stream);
}

jscan_status jscan_step(int64_t d_inner, int64_t d_state, jscan_io io, float* state, const void* x,
                        const void* delta, const float* A, const void* B, const void* C, const float* D,
                        const void* z, void* y, void* stream) {
  return step_impl(1, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, nullptr, nullptr, stream);
}

}  // extern "C"
