// libjscan backward: gradients of the selective scan (jscan_prefill) for
// training, on gfx950.
//
// The forward recurrence (per sequence b, channel d, state n) is
//   h_t = a_t h_{t-1} + dt_t B_t x_t,  a_t = exp(dt_t A),
//   y_t = (C_t . h_t + D x_t) SiLU(z_t)
// ("AI Engineering from Scratch" Jamba lesson, section on the SSM; A real and
// diagonal as in Mamba-1).  Its adjoint, for output gradients dy and dhT,
// runs backwards in time with the same decays:
//   lambda_t = dp_t C_t + mu_{t+1},  mu_t = a_t lambda_t,  mu_L = dhT,
// with dp_t = dy_t SiLU(z_t), and every input gradient is a local product of
// lambda_t, mu_t and the forward state at token t:
//   dx_t     = D dp_t + dt_t (lambda_t . B_t)
//   ddelta_t = x_t (lambda_t . B_t) + sum_n A_n mu_tn h_{t-1,n}
//   dz_t     = dy_t p_t SiLU'(z_t)             (p_t: the pre-gate output)
//   dA_n     = sum_{b,t} dt_t mu_tn h_{t-1,n},   dD = sum_{b,t} dp_t x_t
//   dB_tn    = sum_d lambda_tn dt_t x_t,         dC_tn = sum_d dp_t h_tn
//   dh0      = mu_0.
//
// Work decomposition (one lane per channel, 64 channels per wave, as in the
// forward):
// 1. Records of the forward's chunk-local pass and combine (chunked plans
//    only): the chunk-local state at every sub-chunk boundary and the true
//    state before every forward chunk, from which the forward sweep of
//    step 4 derives its sub-chunk's starting state.
// 2. Chunk-local adjoint (k_adj_local): every chunk but the first runs the
//    adjoint backwards from mu = 0 over its tokens; its result M_c and the
//    chunk's delta sum give the (decay, offset) pair of the chunk.
// 3. k_adj_combine folds the pairs from the last chunk down, seeded with
//    dhT, giving the adjoint that enters each chunk from the later ones.
// 4. Per (chunk, 64 channels): a forward sweep (k_bwd_fwd) from the chunk's
//    starting state writes dz, the dC partial sums and a state checkpoint
//    before every kTok-token block; a reverse sweep (k_bwd_rev) takes the
//    blocks from the last, each as two pieces of PC tokens, the later first:
//    it recomputes a piece's states from the block's checkpoint (into
//    registers) and steps the adjoint back through the piece, writing dx,
//    ddelta and the dB partial sums and accumulating dA.  The recompute of
//    the later piece passes through the states the earlier one needs; two of
//    them are kept in LDS for it.
// 5. Reductions: dB and dC over the 64-channel groups, dA and dD over chunks
//    and sequences (fixed order, so results are deterministic).
// dB_t and dC_t are sums over channels: inside a wave a transposing
// butterfly (permlane swaps and DPP) reduces the 16 values of the 64 lanes
// in 35 instructions, leaving one partial per (group, token, state).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <string>

#include "jscan.h"

#include "common.h"
#include "host.h"

namespace {

using namespace jscan_detail;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int PC = 4;    // a piece: tokens whose states the reverse sweep holds in registers
static_assert(kTok == 2 * PC, "a checkpointed block is two pieces");

// A copy of v the compiler cannot see through.  Recomputed decays would
// otherwise be merged with earlier identical ones and held in registers
// across the whole block, which costs more occupancy than the recompute.
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Sum of v[n] over the 64 lanes of the wave for each n; lane i returns the sum
// for n = i >> 2.  Each step pairs every lane with a partner, keeps half of
// its values and adds the partner's copy of them:
//   permlane32 swap: lanes 0-31 keep n < 8, lanes 32-63 keep n >= 8;
//   permlane16 swap: odd 16-lane rows take n + 4;
//   DPP row_ror:8 (lane i ^ 8 within a row) and row_half_mirror (i ^ 7
//   within 8 lanes) split the last four values over lane bits 3 and 2;
//   two quad_perm adds finish the sum over lane bits 1 and 0.
__device__ __forceinline__ float wave_sum16(const float (&v)[NSTATE], int lane) {
  float r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    r[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  float q[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(r[k]), __float_as_uint(r[k + 4]), false, false);
    q[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
  float s[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) s[k] = (b3 ? q[k + 2] : q[k]) + dpp_mov<0x128>(b3 ? q[k] : q[k + 2]);
  float u = (b2 ? s[1] : s[0]) + dpp_mov<0x141>(b2 ? s[0] : s[1]);
  u += dpp_mov<0xB1>(u);     // quad_perm [1,0,3,2]
  u += dpp_mov<0x4E>(u);     // quad_perm [2,3,0,1]
  return u;
}

// ------------------------------------------------------ chunk-local adjoint
// One lane per channel.  Chunk c >= 1 of sequence b, from its last token
// back to its first with mu = 0 entering: M[b][c][n][d] = mu at the chunk's
// first token, dsum[b][c][d] = sum of delta over the chunk (fp64 sum).  A
// partial last chunk is padded at its end with delta = 0 and dy = 0, which
// keep mu at zero.
template <class T>
__global__ __launch_bounds__(256) void k_adj_local(const T* __restrict__ delta, const float* __restrict__ A,
                                                   const T* __restrict__ Cm, const T* __restrict__ z,
                                                   const T* __restrict__ dy, float* __restrict__ M,
                                                   float* __restrict__ dsum, int64_t L, int64_t d_inner,
                                                   int64_t chunk_len, int n_chunks) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t gbase = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (gbase >= d_inner) return;
  const int c = blockIdx.y + 1;
  const int64_t b = blockIdx.z;
  const int lo = (int)std::min<int64_t>(lane, d_inner - 1 - gbase);
  const int64_t d = gbase + lo;

  float a2[NSTATE], mu[NSTATE];
  const float4* Ap = reinterpret_cast<const float4*>(A + d * NSTATE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = Ap[q];
    a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
    a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
  }
#pragma unroll
  for (int n = 0; n < NSTATE; ++n) mu[n] = 0.0f;
  double dacc = 0.0;

  const int64_t t0 = (int64_t)c * chunk_len;
  const int nt = (int)std::min<int64_t>(chunk_len, L - t0);
  const int64_t row0 = (b * L + t0) * d_inner + gbase;
  const T* drow = delta + row0;
  const T* zrow = z + row0;
  const T* grow = dy + row0;
  const T* crow = Cm + (b * L + t0) * NSTATE;
  const uint32_t lb = (uint32_t)lo * sizeof(T);
  const uint32_t rowb = (uint32_t)(d_inner * sizeof(T));

  auto load_block = [&](int bb, T (&dd)[kTok], T (&zz)[kTok], T (&gg)[kTok]) {
    const int64_t o = (int64_t)bb * d_inner;
    const auto rd = rsrc(drow + o), rz = rsrc(zrow + o), rg = rsrc(grow + o), r0 = rsrc(drow, 0);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const bool real = bb + j < nt;
      const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
      buf_load(dd[j], real ? rd : r0, lb, so);
      buf_load(zz[j], rz, lb, so);
      buf_load(gg[j], real ? rg : r0, lb, so);
    }
  };
  Row<T, NSTATE> Cr;
  auto do_block = [&](int bb, const T (&dd)[kTok], const T (&zz)[kTok], const T (&gg)[kTok]) {
#pragma unroll
    for (int j = kTok - 1; j >= 0; --j) {
      Cr.load(crow + (int64_t)std::min(bb + j, nt - 1) * NSTATE);
      const float dt = widen(dd[j]);
      const float dp = widen(gg[j]) * silu(widen(zz[j]));
      dacc += (double)dt;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) mu[n] = fast_exp2(dt * a2[n]) * fmaf(dp, Cr[n], mu[n]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int last = (nt - 1) / kTok * kTok;
  T dA_[kTok], zA[kTok], gA[kTok], dB_[kTok], zB[kTok], gB[kTok];
  load_block(last, dA_, zA, gA);
  __builtin_amdgcn_s_waitcnt(0);
  for (int base = last; base >= 0; base -= 2 * kTok) {
    load_block(std::max(base - kTok, 0), dB_, zB, gB);
    do_block(base, dA_, zA, gA);
    if (base - kTok < 0) break;
    load_block(std::max(base - 2 * kTok, 0), dA_, zA, gA);
    do_block(base - kTok, dB_, zB, gB);
  }
  if (lo == lane) {
    const int64_t slot = b * n_chunks + c;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) M[(slot * NSTATE + n) * d_inner + d] = mu[n];
    dsum[slot * d_inner + d] = (float)dacc;
  }
}

// ------------------------------------------------------- adjoint carries
// One lane per (b, n, d).  Folds the chunks' pairs from the last chunk down:
// mu <- exp2(A' dsum_c) mu + M_c, seeded with dhT (or 0).  Afterwards slot c
// (c >= 1) of M holds the adjoint entering chunk c - 1 from later tokens.
__global__ __launch_bounds__(256) void k_adj_combine(const float* __restrict__ A, const float* __restrict__ dsum,
                                                     const float* __restrict__ dhT, float* __restrict__ M,
                                                     int64_t d_inner, int n_chunks) {
  constexpr int G = 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t per_seq = d_inner * NSTATE;
  if (i >= per_seq) return;
  const int64_t n = (uint32_t)i / (uint32_t)d_inner;       // 32-bit: i < 16 d_inner <= 2^28
  const int64_t d = i - n * d_inner;
  const float a2 = A[d * NSTATE + n] * kLog2e;
  float mu = dhT ? dhT[(b * d_inner + d) * NSTATE + n] : 0.0f;
  float* Mp = M + (b * n_chunks) * per_seq + i;
  const float* Dp = dsum + (b * n_chunks) * d_inner + d;
  for (int c0 = n_chunks - 1; c0 >= 1; c0 -= G) {
    float mv[G], dv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int c = std::max(c0 - k, 1);
      mv[k] = Mp[(int64_t)c * per_seq];
      dv[k] = Dp[(int64_t)c * d_inner];
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int c = c0 - k;
      if (c >= 1) {
        mu = fmaf(fast_exp2(a2 * dv[k]), mu, mv[k]);
        Mp[(int64_t)c * per_seq] = mu;
      }
    }
  }
}

// ------------------------------------------------------------ main backward
// Grid: (d_inner / 64 groups, chunks, batch); one wave per block.  The two
// sweeps over a chunk are separate kernels so that each gets its own
// register budget.  Padding tokens of a partial last block read delta = 0
// and dy = 0 (empty buffer resource): they change neither the state nor the
// adjoint, and their outputs are not stored.  Lanes clamped onto the last
// channel contribute zero to the channel sums.
struct BwdArgs {
  const void* x; const void* delta; const float* A; const void* B; const void* C; const float* D;
  const void* z; const void* dy;
  const float* h0;        // [b][d][n], may be null: the state before the first (sub-)chunk
  SubRecords rec;         // sub-chunk boundary records and forward chunk starts (chunked plans)
  int64_t fwd_len;        // tokens per forward chunk of the records
  int fwd_chunks;
  const float* Min;       // slot c + 1 = adjoint entering chunk c (chunked plans)
  const float* dhT;
  void* dx; void* ddelta; void* dz;
  float* dBp; float* dCp;  // [b][group][L][16] partial channel sums
  float* dAp; float* dDp;  // [b][chunk][16][d] and [b][chunk][d] partial token sums
  float* dh0;
  float* ck;               // [b][chunk][block][16][d] states before each kTok-token block
  int64_t L, d_inner, chunk_len;
  int n_chunks;
  const int64_t* tag;      // the tag of the prefill whose records `rec` are (saved states), or null
  Tag expect;              // the tag a plain prefill of these sizes and plan writes
};

// False when saved chunk states come from a prefill of other sizes, another
// plan or another variant of the recurrence.  The sweeps then start from NaN,
// so every gradient is NaN rather than silently wrong.
__device__ __forceinline__ bool saved_states_ok(const BwdArgs& a) {
  if (!a.tag) return true;
  bool ok = true;
#pragma unroll
  for (int k = 0; k < kTagWords; ++k) ok = ok && a.tag[k] == a.expect.w[k];
  return ok;
}

// Per-wave coordinates shared by the two sweeps.
struct WaveTile {
  int lane, lo, c, nt, last;
  int64_t g, G, gbase, b, d, t0, row0, blocks;
  float lf;
  uint32_t lb, rowb;
  template <class T>
  __device__ __forceinline__ void init(const BwdArgs& a) {
    lane = threadIdx.x;
    g = blockIdx.x;
    G = gridDim.x;
    gbase = g * 64;
    c = blockIdx.y;
    b = blockIdx.z;
    lo = (int)std::min<int64_t>(lane, a.d_inner - 1 - gbase);
    d = gbase + lo;
    lf = lo == lane ? 1.0f : 0.0f;
    t0 = (int64_t)c * a.chunk_len;
    nt = (int)std::min<int64_t>(a.chunk_len, a.L - t0);
    last = (nt - 1) / kTok * kTok;
    row0 = (b * a.L + t0) * a.d_inner + gbase;
    blocks = (a.chunk_len + kTok - 1) / kTok;
    lb = (uint32_t)lo * sizeof(T);
    rowb = (uint32_t)(a.d_inner * sizeof(T));
  }
};

__device__ __forceinline__ void load_a2(float (&a2)[NSTATE], const float* A, int64_t d) {
  const float4* Ap = reinterpret_cast<const float4*>(A + d * NSTATE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = Ap[q];
    a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
    a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
  }
}

// kTok tokens of the four per-channel streams from block start bb (rows past
// the chunk clamped onto its last token; their delta and dy read 0).
template <class T, int NS>
__device__ __forceinline__ void load_streams(const WaveTile& w, const T* const (&rows)[NS], int bb,
                                             T (&v)[NS][kTok], int delta_slot, int dy_slot,
                                             int64_t d_inner) {
  const int64_t o = (int64_t)bb * d_inner;
  const auto r0 = rsrc(rows[0], 0);
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const auto r = rsrc(rows[k] + o);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const bool real = bb + j < w.nt;
      const uint32_t so = (uint32_t)(std::min(bb + j, w.nt - 1) - bb) * w.rowb;
      buf_load(v[k][j], ((k == delta_slot || k == dy_slot) && !real) ? r0 : r, w.lb, so);
    }
  }
}

// Forward sweep from the chunk's starting state: checkpoints, dz, dC
// partials, dD partial.
template <class T>
__global__ __launch_bounds__(64) void k_bwd_fwd(BwdArgs a, const T* __restrict__ Bm, const T* __restrict__ Cm) {
  WaveTile w;
  w.init<T>(a);
  float a2[NSTATE], h[NSTATE];
  load_a2(a2, a.A, w.d);
  if (a.n_chunks > 1 && w.c > 0) {
    // The true state before sub-chunk c: its boundary's last token lies in
    // forward chunk fc, which started from H[fc] (chunk 0 from h0, where the
    // record is exact); the record holds the chunk-local state there and the
    // delta sum since fc's start.
    const int64_t slot = w.b * a.n_chunks + w.c - 1;
    const int64_t fc = (uint32_t)(w.c * a.chunk_len - 1) / (uint32_t)a.fwd_len;   // 32-bit: below L < 2^31
    const float* S = a.rec.sS + (slot * NSTATE) * a.d_inner + w.d;
    if (fc == 0) {
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = S[(int64_t)n * a.d_inner];
    } else {
      const float lsum = a.rec.sL[slot * a.d_inner + w.d];
      const float* Hc = a.rec.H + ((w.b * a.fwd_chunks + fc) * NSTATE) * a.d_inner + w.d;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n)
        h[n] = fmaf(fast_exp2(a2[n] * lsum), Hc[(int64_t)n * a.d_inner], S[(int64_t)n * a.d_inner]);
    }
  } else {
    const float* hi = a.h0 ? a.h0 + (w.b * a.d_inner + w.d) * NSTATE : nullptr;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) h[n] = hi ? hi[n] : 0.0f;
  }
  const bool ok = saved_states_ok(a);
  if (!ok) {
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) h[n] = __builtin_nanf("");
  }
  const float Dd = a.D[w.d];
  const T* const rows[4] = {static_cast<const T*>(a.delta) + w.row0, static_cast<const T*>(a.x) + w.row0,
                            static_cast<const T*>(a.z) + w.row0, static_cast<const T*>(a.dy) + w.row0};
  T* dzrow = static_cast<T*>(a.dz) + w.row0;
  // B and C rows through the kernel's own restrict parameters, so that they
  // are read with scalar loads
  const T* brow = Bm + (w.b * a.L + w.t0) * NSTATE;
  const T* crow = Cm + (w.b * a.L + w.t0) * NSTATE;
  // checkpoints and partial sums through buffer instructions: wave-uniform
  // bases, the lane's byte offset and a row offset
  const float* ckb = a.ck + ((w.b * a.n_chunks + w.c) * w.blocks * NSTATE) * a.d_inner + w.gbase;
  float* dcb = a.dCp + ((w.b * w.G + w.g) * a.L + w.t0) * NSTATE;
  const uint32_t lb4 = (uint32_t)w.lo * 4, qoff = (uint32_t)(w.lane >> 2) * 4;
  const uint32_t nrow4 = (uint32_t)(a.d_inner * 4);

  float dD = ok ? 0.0f : __builtin_nanf("");
  Row<T, NSTATE> Bc, Bn, Cv;
  auto block = [&](int bb, const T (&v)[4][kTok]) {
    const auto rz = rsrc(dzrow + (int64_t)bb * a.d_inner);
    const auto rdc = rsrc(dcb + (int64_t)bb * NSTATE);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      if (j == 0) {          // checkpoint: the state before the block's first token
        const auto rck = rsrc(ckb + (int64_t)(bb / kTok) * NSTATE * a.d_inner);
#pragma unroll
        for (int n = 0; n < NSTATE; ++n) buf_store(h[n], rck, lb4, (uint32_t)n * nrow4);
      }
      Cv.load(crow + (int64_t)std::min(bb + j, w.nt - 1) * NSTATE);
      Bn.load(brow + (int64_t)std::min(bb + j + 1, w.nt - 1) * NSTATE);
      const float dt = widen(v[0][j]), xv = widen(v[1][j]);
      const float dxv = dt * xv;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dxv * Bc[n]);
      float acc = 0.0f;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) acc = fmaf(Cv[n], h[n], acc);
      const float zv = widen(v[2][j]), gv = widen(v[3][j]);
      const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zv * kLog2e));
      const float sl = zv * sg;
      const float dp = gv * sl;
      const float p = fmaf(Dd, xv, acc);
      dD = fmaf(dp, xv, dD);
      float u[NSTATE];
      const float dpl = dp * w.lf;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) u[n] = dpl * h[n];
      const float sum = wave_sum16(u, w.lane);
      if (bb + j < w.nt) {
        buf_store(to_io(gv * p * sg * (1.0f + zv - sl), T()), rz, w.lb, (uint32_t)j * w.rowb);
        if ((w.lane & 3) == 0) buf_store(sum, rdc, qoff, (uint32_t)j * NSTATE * 4);
      }
      Bc = Bn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One register set: without a second one in flight the kernel fits five
  // waves per SIMD (90 VGPRs instead of 131), which hide the block loads.
  Bc.load(brow);
  for (int base = 0; base < w.nt; base += kTok) {
    T v[4][kTok];
    load_streams(w, rows, base, v, 0, 3, a.d_inner);
    block(base, v);
  }
  if (w.lo == w.lane) a.dDp[(w.b * a.n_chunks + w.c) * a.d_inner + w.d] = dD;
}

// Reverse sweep over the token blocks from the last.  A block is two pieces
// of PC tokens, the later first.  The later piece's states are recomputed
// from the block's checkpoint; that recompute passes through the states
// after the block's first two tokens, which go to LDS, so the earlier piece
// needs one step instead of three.  dx, ddelta, dB partials, dA partial, dh0.
// Three waves per SIMD need at most 168 VGPRs (granule 8 of 512); the bound
// makes the compiler fit them, spilling one dword per block to scratch.
template <class T>
__global__ __launch_bounds__(64, 3) void k_bwd_rev(BwdArgs a, const T* __restrict__ Bm, const T* __restrict__ Cm) {
  WaveTile w;
  w.init<T>(a);
  float a2[NSTATE];
  load_a2(a2, a.A, w.d);
  const float Dd = a.D[w.d];
  const T* const rows[4] = {static_cast<const T*>(a.delta) + w.row0, static_cast<const T*>(a.x) + w.row0,
                            static_cast<const T*>(a.z) + w.row0, static_cast<const T*>(a.dy) + w.row0};
  T* dxrow = static_cast<T*>(a.dx) + w.row0;
  T* ddrow = static_cast<T*>(a.ddelta) + w.row0;
  // B and C rows through the kernel's own restrict parameters, so that they
  // are read with scalar loads
  const T* brow = Bm + (w.b * a.L + w.t0) * NSTATE;
  const T* crow = Cm + (w.b * a.L + w.t0) * NSTATE;
  const float* ckb = a.ck + ((w.b * a.n_chunks + w.c) * w.blocks * NSTATE) * a.d_inner + w.gbase;
  float* dbb = a.dBp + ((w.b * w.G + w.g) * a.L + w.t0) * NSTATE;
  const uint32_t lb4 = (uint32_t)w.lo * 4, qoff = (uint32_t)(w.lane >> 2) * 4;
  const uint32_t nrow4 = (uint32_t)(a.d_inner * 4);

  float mu[NSTATE];
  if (w.c == a.n_chunks - 1) {
    const float* mi = a.dhT ? a.dhT + (w.b * a.d_inner + w.d) * NSTATE : nullptr;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) mu[n] = mi ? mi[n] : 0.0f;
  } else {
    const float* mi = a.Min + ((w.b * a.n_chunks + w.c + 1) * NSTATE) * a.d_inner + w.d;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) mu[n] = mi[(int64_t)n * a.d_inner];
  }
  if (!saved_states_ok(a)) {
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) mu[n] = __builtin_nanf("");
  }
  // LDS indexed (state or quad of states, lane), so that a wave's accesses
  // are consecutive.  dA is carried here (a register accumulator live across
  // the block loop costs the kernel about a hundred VGPRs); st holds, per
  // block, the states after its first and second tokens (4-byte accesses:
  // 16-byte ones need register quads that cost the kernel VGPRs).
  __shared__ float4 dA_lds[4 * 64];
  __shared__ float st_lds[2 * NSTATE * 64];
  auto put = [&](float* base, const float (&h)[NSTATE]) {
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) base[n * 64 + w.lane] = h[n];
  };
  auto get = [&](const float* base, float (&h)[NSTATE]) {
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) h[n] = base[n * 64 + w.lane];
  };
#pragma unroll
  for (int q = 0; q < 4; ++q) dA_lds[q * 64 + w.lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  Row<T, NSTATE> Br, Cv;
  for (int pb = w.last; pb >= 0; pb -= kTok) {
    T v[4][kTok];
    load_streams(w, rows, pb, v, 0, 3, a.d_inner);
    float dps[kTok];                   // dp = dy SiLU(z), so z and dy need not stay live
#pragma unroll
    for (int j = 0; j < kTok; ++j) dps[j] = widen(v[3][j]) * silu(widen(v[2][j]));
    const auto rdb = rsrc(dbb + (int64_t)pb * NSTATE);
    const auto rx = rsrc(dxrow + (int64_t)pb * a.d_inner), rd = rsrc(ddrow + (int64_t)pb * a.d_inner);
    const auto rck = rsrc(ckb + (int64_t)(pb / kTok) * NSTATE * a.d_inner);
    // the state after token pb + j, from the one before it
    auto step = [&](float (&h)[NSTATE], int j) {
      Br.load(brow + (int64_t)std::min(pb + j, w.nt - 1) * NSTATE);
      const float dt = opaque(widen(v[0][j]));
      const float dxv = dt * widen(v[1][j]);
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dxv * Br[n]);
    };
    // the block's checkpoint, read again for each piece rather than held
    auto load_ck = [&](float (&h)[NSTATE]) {
      uint32_t lbh = lb4;
      asm volatile("" : "+v"(lbh));
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) buf_load(h[n], rck, lbh, (uint32_t)n * nrow4);
    };
    // the adjoint back through the piece at hb, given the states before each
    // of its tokens
    auto reverse = [&](int hb, const float (&hp)[PC][NSTATE]) {
      float dAh[NSTATE];
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) dAh[n] = 0.0f;
#pragma unroll
      for (int j = hb + PC - 1; j >= hb; --j) {
        Br.load(brow + (int64_t)std::min(pb + j, w.nt - 1) * NSTATE);
        Cv.load(crow + (int64_t)std::min(pb + j, w.nt - 1) * NSTATE);
        const float dt = opaque(widen(v[0][j])), xv = widen(v[1][j]);
        const float dp = dps[j];
        const float dxl = dt * xv * w.lf;
        float sLB = 0.0f, sAW = 0.0f, u[NSTATE];
#pragma unroll
        for (int n = 0; n < NSTATE; ++n) {
          const float lam = fmaf(dp, Cv[n], mu[n]);
          sLB = fmaf(lam, Br[n], sLB);
          const float m = fast_exp2(dt * a2[n]) * lam;
          mu[n] = m;
          const float wv = m * hp[j - hb][n];
          sAW = fmaf(a2[n], wv, sAW);
          dAh[n] = fmaf(dt, wv, dAh[n]);
          u[n] = lam * dxl;
        }
        const float sum = wave_sum16(u, w.lane);
        if (pb + j < w.nt) {
          const uint32_t so = (uint32_t)j * w.rowb;
          buf_store(to_io(fmaf(Dd, dp, dt * sLB), T()), rx, w.lb, so);
          buf_store(to_io(fmaf(xv, sLB, kLn2 * sAW), T()), rd, w.lb, so);
          if ((w.lane & 3) == 0) buf_store(sum, rdb, qoff, (uint32_t)j * NSTATE * 4);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 t = dA_lds[q * 64 + w.lane];
        t.x += dAh[4 * q]; t.y += dAh[4 * q + 1]; t.z += dAh[4 * q + 2]; t.w += dAh[4 * q + 3];
        dA_lds[q * 64 + w.lane] = t;
      }
    };
    {
      // later piece (tokens PC .. kTok - 1; none past the chunk's end)
      float h[NSTATE];
      load_ck(h);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        step(h, j);
        put(&st_lds[j * NSTATE * 64], h);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pb + PC < w.nt) {
        step(h, 2);
        __builtin_amdgcn_sched_barrier(0);
        step(h, 3);
        __builtin_amdgcn_sched_barrier(0);
        float hp[PC][NSTATE];          // states before each token of the piece
#pragma unroll
        for (int j = 0; j < PC; ++j) {
#pragma unroll
          for (int n = 0; n < NSTATE; ++n) hp[j][n] = h[n];
          if (j + 1 < PC) step(h, PC + j);
          __builtin_amdgcn_sched_barrier(0);
        }
        reverse(PC, hp);
      }
    }
    {
      // earlier piece (tokens 0 .. PC - 1)
      float hp[PC][NSTATE];
      load_ck(hp[0]);
      get(&st_lds[0], hp[1]);
      get(&st_lds[NSTATE * 64], hp[2]);
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) hp[3][n] = hp[2][n];
      step(hp[3], 2);
      __builtin_amdgcn_sched_barrier(0);
      reverse(0, hp);
    }
  }
  float dA[NSTATE];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = dA_lds[q * 64 + w.lane];
    dA[4 * q] = v.x; dA[4 * q + 1] = v.y; dA[4 * q + 2] = v.z; dA[4 * q + 3] = v.w;
  }
  if (w.lo == w.lane) {
    if (w.c == 0 && a.dh0) {
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) a.dh0[(w.b * a.d_inner + w.d) * NSTATE + n] = mu[n];
    }
    const int64_t slot = w.b * a.n_chunks + w.c;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) a.dAp[(slot * NSTATE + n) * a.d_inner + w.d] = dA[n];
  }
}

// dB[b][t][n] and dC[b][t][n]: sums of the G group partials (fixed order).
__global__ __launch_bounds__(256) void k_reduce_bc(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                                   float* __restrict__ dB, float* __restrict__ dC, int64_t L,
                                                   int G) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t per = L * NSTATE;
  if (i >= per) return;
  const float* pb = dBp + (b * G) * per + i;
  const float* pc = dCp + (b * G) * per + i;
  float sb = 0.0f, sc = 0.0f;
  for (int g = 0; g < G; ++g) {
    sb += pb[(int64_t)g * per];
    sc += pc[(int64_t)g * per];
  }
  dB[b * per + i] = sb;
  dC[b * per + i] = sc;
}

// dA[d][n] and dD[d]: sums of the per-(sequence, chunk) partials (fixed order).
__global__ __launch_bounds__(256) void k_reduce_ad(const float* __restrict__ dAp, const float* __restrict__ dDp,
                                                   float* __restrict__ dA, float* __restrict__ dD,
                                                   int64_t d_inner, int64_t slots) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = d_inner * NSTATE;
  if (i >= per) return;
  const int64_t n = (uint32_t)i / (uint32_t)d_inner;       // 32-bit: i < 16 d_inner <= 2^28
  const int64_t d = i - n * d_inner;
  float sa = 0.0f, sd = 0.0f;
  // unrolled so that several loads are in flight; the adds keep their order
#pragma unroll 8
  for (int64_t k = 0; k < slots; ++k) sa += dAp[k * per + i];
  if (n == 0) {
#pragma unroll 8
    for (int64_t k = 0; k < slots; ++k) sd += dDp[k * d_inner + d];
  }
  dA[d * NSTATE + n] = sa;
  if (n == 0) dD[d] = sd;
}

__global__ __launch_bounds__(256) void k_copy_or_zero(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
}

// ------------------------------------------------------------------ host
// Backward workspace: the records a prefill would have left (written here
// only when they are recomputed; the backward's chunks are the plan's
// sub-chunks), then the adjoint carries, state checkpoints and partial sums.
struct BwdLayout {
  size_t fwd, M, dsum, ck, dBp, dCp, dAp, dDp, total;
};

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p) {
  BwdLayout w{};
  if (batch <= 0 || L <= 0 || d_inner <= 0) return w;
  const size_t B = (size_t)batch, C = (size_t)p.subs, Dn = (size_t)d_inner;
  const size_t G = (size_t)((d_inner + 63) / 64);
  const size_t blocks = (size_t)((p.sub_len + kTok - 1) / kTok);
  // the size of a prefill's workspace (its records and RMSNorm region), so a
  // backward reusing one needs jscan_prefill_workspace_size() bytes less
  w.fwd = ws_layout(batch, L, d_inner, p).total + rms_bytes(batch * L);
  if (p.subs > 1) {
    w.M = round_up(B * C * NSTATE * Dn * 4);
    w.dsum = round_up(B * C * Dn * 4);
  }
  w.ck = round_up(B * C * blocks * NSTATE * Dn * 4);
  w.dBp = round_up(B * G * (size_t)L * NSTATE * 4);
  w.dCp = w.dBp;
  w.dAp = round_up(B * C * NSTATE * Dn * 4);
  w.dDp = round_up(B * C * Dn * 4);
  w.total = w.fwd + w.M + w.dsum + w.ck + w.dBp + w.dCp + w.dAp + w.dDp;
  return w;
}

template <class T>
jscan_status run_backward(int64_t batch, int64_t L, int64_t d_inner, jscan_io io, const void* x, const void* delta,
                          const float* A, const void* B, const void* C, const float* D, const void* z,
                          const float* h0, const void* dy, const float* dhT, void* dx, void* ddelta, void* dz,
                          float* dA, float* dB, float* dC, float* dD, float* dh0, char* ws,
                          const char* saved, const Plan& p, hipStream_t st) {
  const BwdLayout w = bwd_layout(batch, L, d_inner, p);
  // The forward sweep derives each sub-chunk's starting state from the
  // records a prefill left in its workspace (`saved`) or from records
  // recomputed into this one (which need their region only without saved
  // ones and with more than one sub-chunk).
  char* q = ws;
  char* rec = !saved && p.subs > 1 ? q : nullptr;
  if (rec) q += w.fwd;
  float* M = reinterpret_cast<float*>(q); q += w.M;
  float* dsum = reinterpret_cast<float*>(q); q += w.dsum;
  float* ck = reinterpret_cast<float*>(q); q += w.ck;
  float* dBp = reinterpret_cast<float*>(q); q += w.dBp;
  float* dCp = reinterpret_cast<float*>(q); q += w.dCp;
  float* dAp = reinterpret_cast<float*>(q); q += w.dAp;
  float* dDp = reinterpret_cast<float*>(q);
  const int G = (int)((d_inner + 63) / 64);
  const int chunks = p.subs;
  hipError_t e;
  jscan_status s;

  SubRecords recs{};
  if (chunks > 1) {
    if ((s = backward_records(io, batch, L, d_inner, x, delta, A, B, h0, rec, saved, p, st, &recs)) != JSCAN_OK)
      return s;
    dim3 g1((unsigned)((d_inner + 255) / 256), (unsigned)(chunks - 1), (unsigned)batch);
    hipLaunchKernelGGL((k_adj_local<T>), g1, dim3(256), 0, st, static_cast<const T*>(delta), A,
                       static_cast<const T*>(C), static_cast<const T*>(z), static_cast<const T*>(dy), M, dsum, L,
                       d_inner, p.sub_len, chunks);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "adjoint chunk launch");
    dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
    hipLaunchKernelGGL(k_adj_combine, g2, dim3(256), 0, st, A, dsum, dhT, M, d_inner, chunks);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "adjoint combine launch");
  }
  const BwdArgs args{x, delta, A, B, C, D, z, dy, h0, recs, p.chunk_len, p.chunks, M, dhT, dx, ddelta, dz, dBp, dCp,
                     dAp, dDp, dh0, ck, L, d_inner, p.sub_len, chunks,
                     saved ? reinterpret_cast<const int64_t*>(saved) : nullptr, make_tag(batch, L, d_inner, p, 0)};
  dim3 g3((unsigned)G, (unsigned)chunks, (unsigned)batch);
  hipLaunchKernelGGL((k_bwd_fwd<T>), g3, dim3(64), 0, st, args, static_cast<const T*>(B), static_cast<const T*>(C));
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "backward forward-sweep launch");
  hipLaunchKernelGGL((k_bwd_rev<T>), g3, dim3(64), 0, st, args, static_cast<const T*>(B), static_cast<const T*>(C));
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "backward reverse-sweep launch");
  dim3 g4((unsigned)((L * NSTATE + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(k_reduce_bc, g4, dim3(256), 0, st, dBp, dCp, dB, dC, L, G);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "dB/dC reduce launch");
  hipLaunchKernelGGL(k_reduce_ad, dim3((unsigned)((d_inner * NSTATE + 255) / 256)), dim3(256), 0, st, dAp, dDp, dA,
                     dD, d_inner, batch * (int64_t)chunks);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "dA/dD reduce launch");
  return JSCAN_OK;
}

// jscan_backward (saved = false) and jscan_backward_saved (saved = true:
// the chunk starting states come from the workspace of the prefill call).
jscan_status backward_impl(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                           const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* h0, const void* dy, const float* dhT,
                           void* dx, void* ddelta, void* dz, float* dA, float* dB, float* dC, float* dD,
                           float* dh0, bool saved, const void* prefill_ws, size_t prefill_ws_bytes,
                           void* workspace, size_t workspace_bytes, void* stream) {
  t_last_error.clear();
  jscan_status s = check_common(d_state, io);
  if (s != JSCAN_OK) return s;
  if (!sizes_ok(batch, L, d_inner)) return fail(JSCAN_ERR_SHAPE, "sizes must be >= 0 and fit 64-bit byte counts");
  const bool work = batch > 0 && L > 0 && d_inner > 0;
  if (work && (!x || !delta || !B || !C || !z || !dy || !dx || !ddelta || !dz || !dB || !dC))
    return fail(JSCAN_ERR_NULL, "x, delta, B, C, z, dy, dx, ddelta, dz, dB and dC are required");
  if (d_inner > 0 && (!A || !D || !dA || !dD)) return fail(JSCAN_ERR_NULL, "A, D, dA and dD are required");
  const void* ptrs[] = {x, delta, A, B, C, D, z, h0, dy, dhT, dx, ddelta, dz, dA, dB, dC, dD, dh0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)batch * (size_t)L * (size_t)d_inner * es;
  const size_t rowb = (size_t)batch * (size_t)L * NSTATE * es;
  const size_t row4 = (size_t)batch * (size_t)L * NSTATE * 4;
  const size_t stb = (size_t)batch * (size_t)d_inner * NSTATE * 4;
  const size_t pd = (size_t)d_inner * NSTATE * 4;
  const Plan plan = choose_plan(batch, L, d_inner);
  const BwdLayout bl = bwd_layout(batch, L, d_inner, plan);
  // With saved chunk states the front of the workspace (the prefill's part) is not needed.
  const bool use_saved = saved && work && plan.subs > 1;
  // a saved-state call needs jscan_prefill_workspace_size() bytes less in every plan
  const size_t need = saved ? bl.total - bl.fwd : bl.total;
  // the prefill's workspace: jscan_prefill_workspace_size() bytes (records and RMSNorm region)
  const size_t pws_need = ws_layout(batch, L, d_inner, plan).total + rms_bytes(batch * L);
  if (use_saved && !prefill_ws)
    return fail(JSCAN_ERR_NULL, "this plan runs in chunks: the prefill's workspace is required");
  if (use_saved && !aligned16(prefill_ws))
    return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  if (use_saved && prefill_ws_bytes < pws_need)
    return fail(JSCAN_ERR_WORKSPACE, "prefill workspace smaller than jscan_prefill_workspace_size()");
  const Range in[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {dy, tok, "dy"}, {B, rowb, "B"},
                      {C, rowb, "C"}, {A, pd, "A"}, {D, (size_t)d_inner * 4, "D"}, {h0, stb, "h0"},
                      {dhT, stb, "dhT"}, {use_saved ? prefill_ws : nullptr, use_saved ? pws_need : 0,
                                          "prefill workspace"}};
  const Range out[] = {{dx, tok, "dx"}, {ddelta, tok, "ddelta"}, {dz, tok, "dz"}, {dA, pd, "dA"},
                       {dB, row4, "dB"}, {dC, row4, "dC"}, {dD, (size_t)d_inner * 4, "dD"}, {dh0, stb, "dh0"},
                       {workspace, workspace ? need : 0, "workspace"}};
  if ((s = check_ranges(in, (int)(sizeof(in) / sizeof(in[0])), out, (int)(sizeof(out) / sizeof(out[0])))) !=
      JSCAN_OK)
    return s;
  if (workspace && workspace_bytes < need)
    return fail(JSCAN_ERR_WORKSPACE, saved ? "workspace smaller than jscan_backward_workspace_size() - "
                                                 "jscan_prefill_workspace_size()"
                                               : "workspace smaller than jscan_backward_workspace_size()");

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!work) {
    // Nothing to scan: parameter gradients are zero and dh0 = dhT (or 0).
    if (d_inner > 0) {
      hipLaunchKernelGGL(k_reduce_ad, dim3((unsigned)((d_inner * NSTATE + 255) / 256)), dim3(256), 0, st,
                         nullptr, nullptr, dA, dD, d_inner, (int64_t)0);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "zero-fill launch");
    }
    if (dh0 && batch > 0 && d_inner > 0) {
      const int64_t n = batch * d_inner * NSTATE;
      hipLaunchKernelGGL(k_copy_or_zero, dim3(copy_grid(n)), dim3(256), 0, st, dhT, dh0, n);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "dh0 copy launch");
    }
    return JSCAN_OK;
  }
  char* ws = static_cast<char*>(workspace);
  bool owned = false;
  if (!ws) {
    if ((e = hipMallocAsync(reinterpret_cast<void**>(&ws), need, st)) != hipSuccess)
      return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }
  const char* pw = use_saved ? static_cast<const char*>(prefill_ws) : nullptr;
  s = io == JSCAN_IO_BF16
          ? run_backward<uint16_t>(batch, L, d_inner, io, x, delta, A, B, C, D, z, h0, dy, dhT, dx, ddelta, dz,
                                   dA, dB, dC, dD, dh0, ws, pw, plan, st)
          : run_backward<float>(batch, L, d_inner, io, x, delta, A, B, C, D, z, h0, dy, dhT, dx, ddelta, dz, dA,
                                dB, dC, dD, dh0, ws, pw, plan, st);
  if (owned) {
    e = hipFreeAsync(ws, st);
    if (s == JSCAN_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync(workspace)");
  }
  return s;
}

}  // namespace

// ================================================================ C ABI
extern "C" {

size_t jscan_backward_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io) {
  (void)io;
  if (d_state != NSTATE || !sizes_ok(batch, L, d_inner)) return 0;
  return bwd_layout(batch, L, d_inner, choose_plan(batch, L, d_inner)).total;
}

jscan_status jscan_backward(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                            const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const float* h0, const void* dy, const float* dhT,
                            void* dx, void* ddelta, void* dz, float* dA, float* dB, float* dC, float* dD,
                            float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, dy, dhT, dx, ddelta, dz, dA,
                       dB, dC, dD, dh0, false, nullptr, 0, workspace, workspace_bytes, stream);
}

jscan_status jscan_backward_saved(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                  const void* x, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* h0, const void* dy,
                                  const float* dhT, void* dx, void* ddelta, void* dz, float* dA, float* dB,
                                  float* dC, float* dD, float* dh0, const void* prefill_workspace,
                                  size_t prefill_workspace_bytes, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return backward_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, dy, dhT, dx, ddelta, dz, dA,
                       dB, dC, dD, dh0, true, prefill_workspace, prefill_workspace_bytes, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
