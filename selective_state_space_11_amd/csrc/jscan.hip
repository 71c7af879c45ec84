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
// * Lanes map to channels: a wave covers 64 consecutive channels and all 16
//   states of each, so each per-token load of x, delta and z is one coalesced
//   128-byte row segment.  The state stays in VGPRs for the whole call.
//   Because every lane of a wave needs the same per-token rows B_t and C_t,
//   they are read with scalar loads into SGPRs (bf16 pairs stay packed and
//   are widened by a scalar shift or mask) and fed to the VALU as scalar
//   operands, with no LDS traffic and no VGPRs.
// * The scan is bound by the fp32 VALU, not by HBM: per channel-token it
//   moves 8 bytes but issues about 93 VALU instructions (16 decays exp2 and
//   4 plain operations per state, plus the epilogue).  The chip therefore
//   needs every SIMD busy, and at batch 1 the 8192 channels are only 128
//   waves: the sequence is cut into chunks scanned in parallel.
// * Chunked prefill, two passes and a combine:
//   - pass 1 scans every chunk from a zero state (chunk 0 from h0) and
//     records the chunk-local state and the delta sum at the end of each
//     sub-chunk (the last record of a chunk is its end).  The part of a later
//     chunk's state it misses is the carried-in state decayed by
//     exp(A * sum delta), at most exp2(A'max * sum delta) * |h_start| for the
//     slowest state: once sum delta reaches 24 / |A'max| in every lane of the
//     wave that is below fp32 resolution, so pass 1 scans state-only up to
//     that token and writes y from it on (chunk 0, being exact, writes all);
//   - the combine folds the chunks' (decay, end state) pairs in order,
//     h <- exp2(A' * sum delta) * h + S, giving each chunk's true starting
//     state and the final state;
//   - pass 2 rescans each later chunk from its true starting state and writes
//     y, until the same bound, now with the true |h_start|, is below fp32
//     resolution of the state in every lane of the wave, and never before the
//     token from which pass 1 wrote y.  The carried part only decays when
//     A <= 0 and delta >= 0, so a wave that sees A > 0, or a chunk with a
//     negative time step, rescans its whole chunk.
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
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "jscan.h"

#include "common.h"
#include "host.h"

namespace jscan_detail {

enum ScanMode : int {
  kWhole = 0,    // one chunk per sequence: from h0, writes y, hT (and the conv history)
  kLocal = 1,    // pass 1: from zero (chunk 0 from h0), writes y and the sub-chunk records
  kFix = 2,      // pass 2: chunks >= 1 from their true starting state until the carry has decayed
};

// A carried difference below this fraction of the lane's largest state
// magnitude no longer changes the state in fp32.
constexpr float kSettled = 0x1p-24f;

// Waves per SIMD the main scan's register allocation is held to (the second
// __launch_bounds__ argument, amdgpu-waves-per-eu; 1 = no bound).  A SIMD
// lane has 512 VGPRs in granules of 8, so 4 waves allow 128.  The bf16
// trapezoidal scan needs 129 without a bound (3 waves); held to 4 waves it
// fits 121 without spilling VGPRs and runs its 64K prefill about 6% faster.
template <class T, bool CONV, bool SP, bool TR, bool RMS, int MODE>
constexpr int scan_waves() { return sizeof(T) == 2 && (TR || MODE != kWhole) ? 4 : 1; }

// One float from a wave-uniform address, as a scalar load.
__device__ __forceinline__ float load_uniform(const float* p) { return __uint_as_float(*uniform_ptr<uint32_t>(p)); }

__device__ __forceinline__ void load_a2(float (&a2)[NSTATE], const float* A, int64_t d) {
  const float4* Ap = reinterpret_cast<const float4*>(A + d * NSTATE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = Ap[q];
    a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
    a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
  }
}

// A record: the lane's 16 chunk-local states (state-major, S[slot][n][d])
// and the delta sum since the chunk start, through buffer stores (wave-uniform
// base at channel gbase, the lane's byte offset lb4 and a row offset), which
// cost no VGPRs for addresses.
__device__ __forceinline__ void write_record(float* __restrict__ S, float* __restrict__ Ls,
                                             const float (&h)[NSTATE], double dacc, int64_t slot,
                                             int64_t d_inner, int64_t gbase, uint32_t lb4) {
  const auto rs = rsrc(S + slot * NSTATE * d_inner + gbase);
  const uint32_t row = (uint32_t)(d_inner * 4);
#pragma unroll
  for (int n = 0; n < NSTATE; ++n) buf_store(h[n], rs, lb4, (uint32_t)n * row);
  buf_store((float)dacc, rsrc(Ls + slot * d_inner + gbase), lb4, 0);
}

// Where the records of a chunk go.  After the block ending at chunk-local
// token `end`: the chunk's end record when the block ends the chunk, and the
// record of sub-chunk s when the block ends at the sub-chunk boundary
// (s + 1) * sub_len inside the sequence.
// The next sub-chunk boundary after a wave's position and the record slot it
// fills.  Chunk starts and sub-chunk lengths are multiples of the block
// length, so every boundary is a block end; the cursor moves on by one
// sub-chunk at each (no division in the token loop).
struct SubCursor {
  int next;        // chunk-local token of the next boundary (INT32_MAX: none)
  int slot;        // its record slot
  int step;        // the sub-chunk length
  bool seq_end;    // the chunk ends the sequence (no boundary at its end)
};

struct Records {
  float* eS; float* eL;        // [b][chunks][16][d], [b][chunks][d]
  float* sS; float* sL;        // [b][subs][16][d], [b][subs][d], or null (one sub-chunk)
  int64_t sub_len;
  int chunks, subs;
  __device__ __forceinline__ SubCursor cursor(int64_t t0, int nt, int64_t L, int64_t b) const {
    if (!sS) return SubCursor{INT32_MAX, 0, 0, false};
    const int64_t k = t0 / sub_len + 1;            // the first boundary after t0
    return SubCursor{(int)(k * sub_len - t0), (int)(b * subs + k - 1), (int)sub_len, t0 + nt >= L};
  }
  // After the block ending at chunk-local token `end` (exclusive).
  __device__ __forceinline__ void after_block(int end, int nt, int64_t b, int c, const float (&h)[NSTATE],
                                              double dacc, int64_t d_inner, int64_t gbase, bool real,
                                              uint32_t lb4, SubCursor& cur) const {
    if (end == cur.next) {
      if (real && !(end >= nt && cur.seq_end)) write_record(sS, sL, h, dacc, cur.slot, d_inner, gbase, lb4);
      cur.next += cur.step;
      ++cur.slot;
    }
    if (end >= nt && real) write_record(eS, eL, h, dacc, b * chunks + c, d_inner, gbase, lb4);
  }
};

// Issue priority by progress through the chunk.  A SIMD's arbiter issues the
// oldest ready wave first, so among waves with the same work the first
// dispatched finish far ahead of the last, and the SIMD then runs the last
// stretch with fewer waves and worse latency hiding.  Lowering a wave's
// priority (s_setprio, 3 = highest) as it passes half, three quarters and
// nine tenths of its tokens lets the waves behind catch up, so they all
// finish close together.  Pass 2 takes it too: when the carry settles early
// its waves stay at the top priority, and when decay is slow it rescans
// whole chunks, where the balancing makes it about 8% faster.
struct ProgressPrio {
  int t1, t2, t3;
  __device__ __forceinline__ explicit ProgressPrio(int nt)
      : t1(nt / 2), t2((int)((int64_t)nt * 3 / 4)), t3((int)((int64_t)nt * 9 / 10)) {}
  __device__ __forceinline__ void set(int done) const {
    if (done < t1) __builtin_amdgcn_s_setprio(3);
    else if (done < t2) __builtin_amdgcn_s_setprio(2);
    else if (done < t3) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
};

// ---------------------------------------- chunk-local states (backward only)
// The state half of pass 1 for the plain recurrence, for a backward that has
// to recompute the records: one lane per channel, all 16 states, chunk c of
// sequence b from zero (chunk 0 from h0).  Its arithmetic is pass 1's,
// operation for operation, so both write identical records.
template <class T>
__global__ __launch_bounds__(256) void k_chunk_state(const T* __restrict__ x, const T* __restrict__ delta,
                                                     const float* __restrict__ A, const T* __restrict__ Bm,
                                                     const float* __restrict__ h0, Records rec, int64_t L,
                                                     int64_t d_inner, int64_t chunk_len) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t gbase = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (gbase >= d_inner) return;                       // whole wave past the end
  const int c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lo = (int)std::min<int64_t>(lane, d_inner - 1 - gbase);
  const int64_t d = gbase + lo;

  float a2[NSTATE], h[NSTATE];
  load_a2(a2, A, d);
  const float* hi = c == 0 && h0 ? h0 + (b * d_inner + d) * NSTATE : nullptr;
#pragma unroll
  for (int n = 0; n < NSTATE; ++n) h[n] = hi ? hi[n] : 0.0f;
  double dacc = 0.0;

  const int64_t t0 = (int64_t)c * chunk_len;
  const int nt = (int)std::min<int64_t>(chunk_len, L - t0);
  const T* xrow = x + (b * L + t0) * d_inner + gbase;
  const T* drow = delta + (b * L + t0) * d_inner + gbase;
  const T* brow = Bm + (b * L + t0) * NSTATE;
  const uint32_t lb = (uint32_t)lo * sizeof(T);
  const uint32_t rowb = (uint32_t)(d_inner * sizeof(T));
  const int last = (nt - 1) / kTok * kTok;
  const ProgressPrio prio(nt);
  SubCursor cur = rec.cursor(t0, nt, L, b);

  auto load_block = [&](int bb, T (&dd)[kTok], T (&xx)[kTok]) {
    const int64_t o = (int64_t)bb * d_inner;
    const auto rd = rsrc(drow + o), rx = rsrc(xrow + o), r0 = rsrc(drow, 0);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
      buf_load(dd[j], bb + j < nt ? rd : r0, lb, so);
      buf_load(xx[j], rx, lb, so);
    }
  };
  Row<T, NSTATE> Bc, Bn;
  auto do_block = [&](int bb, const T (&dd)[kTok], const T (&xx)[kTok]) {
    float bsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      Bn.load(brow + (int64_t)std::min(bb + j + 1, nt - 1) * NSTATE);
      const float dt = widen(dd[j]);
      const float dx = dt * widen(xx[j]);
      bsum += dt;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dx * Bc[n]);
      Bc = Bn;
      __builtin_amdgcn_sched_barrier(0);
    }
    dacc += (double)bsum;
    rec.after_block(bb + kTok, nt, b, c, h, dacc, d_inner, gbase, lo == lane, (uint32_t)lo * 4, cur);
  };
  T dA[kTok], xA[kTok], dB[kTok], xB[kTok];
  load_block(0, dA, xA);
  Bc.load(brow);
  __builtin_amdgcn_s_waitcnt(0);
  for (int base = 0; base < nt; base += 2 * kTok) {
    prio.set(base);
    load_block(std::min(base + kTok, last), dB, xB);
    do_block(base, dA, xA);
    if (base + kTok >= nt) break;
    load_block(std::min(base + 2 * kTok, last), dA, xA);
    do_block(base + kTok, dB, xB);
  }
}

// ------------------------------------------------------------ carry combine
// One lane per (b, n, d), d fastest.  Folds the forward chunks' (P, S) pairs
// in sequence order, h <- P * h + S with P = exp2(A' * delta sum) and S the
// chunk's end record, starting from chunk 0's (which began at h0);
// H[b][c][n][d] = the state before chunk c, and the state after the last
// chunk is hT.  Also writes the conv history after the sequence (the last
// width - 1 raw x, or history values for a short sequence) and the
// workspace tag.
template <class T>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ A, const float* __restrict__ eS,
                                                 const float* __restrict__ eL, float* __restrict__ H,
                                                 float* __restrict__ hT, int64_t d_inner, int chunks,
                                                 const T* __restrict__ x, int64_t L, ProArgs pa,
                                                 int64_t* __restrict__ tag_out, Tag tag) {
  constexpr int G = 16;                // chunks whose loads are in flight together
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (tag_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kTagWords)
    tag_out[threadIdx.x] = tag.w[threadIdx.x];
  const int64_t per_seq = d_inner * NSTATE;
  if (i >= per_seq) return;
  const int64_t n = (uint32_t)i / (uint32_t)d_inner;       // 32-bit: i < 16 d_inner <= 2^28
  const int64_t d = i - n * d_inner;
  const float a2 = A[d * NSTATE + n] * kLog2e;
  const float* Sp = eS + (b * chunks) * per_seq + i;
  const float* Lp = eL + (b * chunks) * d_inner + d;
  float* Hp = H + (b * chunks) * per_seq + i;
  float h = Sp[0];
  for (int c0 = 1; c0 < chunks; c0 += G) {
    float sv[G], lv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int c = std::min(c0 + k, chunks - 1);
      sv[k] = Sp[(int64_t)c * per_seq];
      lv[k] = Lp[(int64_t)c * d_inner];
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (c0 + k < chunks) {
        Hp[(int64_t)(c0 + k) * per_seq] = h;
        h = fmaf(fast_exp2(a2 * lv[k]), h, sv[k]);
      }
    }
  }
  if (hT) hT[(b * d_inner + d) * NSTATE + n] = h;
  // Conv history after the sequence, by the lane of state 0 of each channel,
  // slot by slot: with an in-place history (hist_out == hist) slot j is read
  // from slot j + L >= j, before that slot is written.
  if (pa.hist_out && n == 0) {
    for (int j = 0; j < pa.width - 1; ++j) {
      const int64_t pos = L - (pa.width - 1) + j;
      const int64_t k = (pa.width - 1) + pos;
      const float v = pos >= 0 ? widen(x[(b * L + pos) * d_inner + d])
                               : (pa.hist && k >= 0 ? pa.hist[(b * (pa.width - 1) + k) * d_inner + d] : 0.0f);
      pa.hist_out[(b * (pa.width - 1) + j) * d_inner + d] = v;
    }
  }
}

// ----------------------------------------------------------------- main scan
// Extra arguments of the main scan (pointers into the workspace).
struct ScanAux {
  const float* h0;        // [b][d][n] (kWhole, and chunk 0 in kLocal), may be null
  float* hT;              // kWhole
  Records rec;            // kLocal: chunk-end and sub-chunk records
  int32_t* neg;           // kLocal writes, kFix reads: a negative time step in [b][chunk][d]
  int32_t* from;          // progress records [b][chunk][group][2]: the first token pass 1 wrote y for
                          // (kLocal writes, kFix reads) and the token where pass 2 stopped (kFix)
  const float* H;         // kFix: chunk starting states [b][chunk][n][d]
  int64_t L, d_inner, chunk_len;
  int chunks, groups;
};

// Grid: (ceil(d_inner / 64), chunks (kFix: chunks - 1), batch); one wave per
// block, owning all 16 states of its 64 channels for the block's chunk.
//
// Tokens go in blocks of kTok, the next block's loads issued before the
// current block is computed.  A chunk's last block may be partial: its
// missing tokens are loaded clamped onto the last token with delta = 0, so
// they leave the state bit-for-bit unchanged (exp2(0) = 1, input term
// 0 * x * B = 0 for finite x and B) and their output equals the last token's,
// which they store again to the same address.  Every block therefore runs the
// same branch-free code.
template <class T, bool CONV, bool SP, bool TR, bool RMS, int MODE>
__global__ __launch_bounds__(64, (scan_waves<T, CONV, SP, TR, RMS, MODE>())) void k_scan(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dw, const T* __restrict__ z,
    T* __restrict__ y, ScanAux aux, ProArgs pa) {
  static_assert(!(CONV && TR), "the trapezoidal form takes no outer convolution");
  static_assert(!(RMS && TR), "the trapezoidal form takes no RMSNorm");
  using RT = std::conditional_t<RMS, float, T>;     // B and C rows: fp32 after RMSNorm
  const int lane = threadIdx.x;
  const int64_t L = aux.L, d_inner = aux.d_inner;
  const int64_t gbase = (int64_t)blockIdx.x * 64;
  const int c = MODE == kFix ? (int)blockIdx.y + 1 : (int)blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lo = (int)std::min<int64_t>(lane, d_inner - 1 - gbase);
  const int64_t d = gbase + lo;

  float a2[NSTATE], h[NSTATE];
  load_a2(a2, A, d);
  bool can_exit = true;
  // kLocal: chunk 0 (from the true h0) writes all its y; a later chunk starts
  // writing y at the block after which sum delta >= settle_sum in every lane
  bool emit = MODE != kLocal || blockIdx.y == 0;
  int emit_from = 0;
  double settle_sum = 0.0;
  if constexpr (MODE == kLocal) {
    float a2max = a2[0];
#pragma unroll
    for (int n = 1; n < NSTATE; ++n) a2max = fmaxf(a2max, a2[n]);
    settle_sum = a2max < 0.0f ? 24.0 / -(double)a2max : __builtin_inf();
  }
  // kFix: the first token from which pass 1 wrote y for this wave's channels
  // progress record of this wave's (sequence, chunk, channel group): the
  // token from which pass 1 wrote y, and the token where pass 2 stopped
  int32_t* const prog = MODE == kWhole ? nullptr : aux.from + 2 * ((b * aux.chunks + c) * aux.groups + blockIdx.x);
  const int fix_from = MODE == kFix ? prog[0] : 0;
  // kFix: the carry pass 1 missed is exp(A * sum delta) * h_start, at most
  // exp2(fix_a2 * sum delta) * fix_h with the slowest state's A' and the
  // largest |h_start|.
  float fix_a2 = -__builtin_inff(), fix_h = 0.0f;
  if constexpr (MODE == kFix) {
    const float* hi = aux.H + ((b * aux.chunks + c) * NSTATE) * d_inner + d;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) {
      h[n] = hi[(int64_t)n * d_inner];
      fix_h = fmaxf(fix_h, fabsf(h[n]));
      fix_a2 = fmaxf(fix_a2, a2[n]);
      can_exit = can_exit && a2[n] <= 0.0f;
    }
    can_exit = can_exit && aux.neg[(b * aux.chunks + c) * d_inner + d] == 0;
  } else {
    const float* hi = (MODE == kWhole || c == 0) && aux.h0 ? aux.h0 + (b * d_inner + d) * NSTATE : nullptr;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) h[n] = hi ? hi[n] : 0.0f;
  }
  const float Dd = Dw[d];

  const int64_t t0 = (int64_t)c * aux.chunk_len;
  const int nt = (int)std::min<int64_t>(aux.chunk_len, L - t0);   // >= 1 for every chunk
  SubCursor sub_cur{};               // kLocal: the next sub-chunk record
  if constexpr (MODE == kLocal) sub_cur = aux.rec.cursor(t0, nt, L, b);
  const int64_t row0 = (b * L + t0) * d_inner + gbase;
  const T* xrow = x + row0;
  const T* drow = delta + row0;
  const T* zrow = z + row0;
  T* yrow = y + row0;
  const RT* brow;
  const RT* crow;
  if constexpr (RMS) {
    brow = pa.rms_B + (b * L + t0) * NSTATE;
    crow = pa.rms_C + (b * L + t0) * NSTATE;
  } else {
    brow = Bm + (b * L + t0) * NSTATE;
    crow = Cm + (b * L + t0) * NSTATE;
  }
  // RMSNorm: delta * w[d] * s[t], s of the next token loaded during the token before it
  const float* srow = RMS ? pa.rms_s + b * L + t0 : nullptr;
  const float wdt = RMS && pa.rms_w ? pa.rms_w[d] : 1.0f;
  float s_cur = 1.0f, s_next = 1.0f;
  auto raw_dt = [&](T v) {
    float r = widen(v);
    if constexpr (RMS) r = r * wdt * s_cur;
    return r;
  };

  const uint32_t lb = (uint32_t)lo * sizeof(T);      // lane byte offset within a row
  const uint32_t rowb = (uint32_t)(d_inner * sizeof(T));
  Prologue<CONV, SP> pro;
  pro.init(pa, d);
  pro.start(pa, pa.hist, x, b, L, d_inner, t0, d);
  // Trapezoidal form: the scan runs on the shifted state g (see trap_seed);
  // chunk 0 starts from h0 + w_0 B_prev, later chunks from the combine's g.
  const T* lrow = TR && pa.lam ? static_cast<const T*>(pa.lam) + row0 : drow;
  const float lam_add = TR && !pa.lam ? 0.5f : 0.0f;      // a missing lam reads 0 through the empty resource
  if constexpr (TR && MODE != kFix) {
    if (c == 0) trap_seed(h, pa, pro, delta, b, L, d_inner, d, 0);
  }

  // Loads of token block bb.  Rows past the chunk's end are clamped onto its
  // last token, and their delta is read through an empty resource (0).  With
  // TR also: delta and lam of the token after the block (0 past the
  // sequence's end), and for the block's C_t . B_t products lane l's pair of
  // states 2 (l & 7) + {0, 1} of token bb + (l >> 3), B and C.
  auto load_block = [&](int bb, T (&dq)[kTok], T (&xx)[kTok], T (&zz)[kTok], T (&ll)[kTok], T& dn, T& ln,
                        Pair<T>& pb, Pair<T>& pc) __attribute__((always_inline)) {
    const int64_t o = (int64_t)bb * d_inner;
    const auto rd = rsrc(drow + o), rx = rsrc(xrow + o), rz = rsrc(zrow + o), r0 = rsrc(drow, 0);
    const auto rl = TR && pa.lam ? rsrc(lrow + o) : r0;
    // Token by token, so that a token's loads are consumed in issue order and
    // its wait covers only the loads before it (the barrier keeps the
    // compiler from regrouping them by stream).
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
      buf_load(dq[j], bb + j < nt ? rd : r0, lb, so);
      buf_load(xx[j], rx, lb, so);
      buf_load(zz[j], rz, lb, so);
      if constexpr (TR) buf_load(ll[j], rl, lb, so);
      __builtin_amdgcn_sched_barrier(0);
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
  };

  // A token's B row is loaded during the token before it (right after that
  // token's state update, into the same registers); C is needed only after
  // the state updates, so it is loaded at the token's start.
  Row<RT, NSTATE> Bc, Cv;
  double dacc = 0.0;                 // kLocal: delta sum since the chunk start
  float fsum = 0.0f;                 // kFix: delta sum since the chunk start
  uint32_t negbits = 0;              // kLocal: OR of the time steps' bits (sign bit)
  // y of token bb + j (padding tokens map onto the last token's address and
  // store the identical value again).  With a convolution, a padding token's
  // input differs (its history has shifted), so only real tokens store.
  auto finish = [&](__amdgpu_buffer_rsrc_t ry, int bb, int j, float acc, float xv, float zv) {
    const uint32_t so = (uint32_t)(std::min(bb + j, nt - 1) - bb) * rowb;
    if (!CONV || bb + j < nt) buf_store(to_io(fmaf(Dd, xv, acc) * silu(zv), T()), ry, lb, so);
  };
  // Returns true (kFix) once the carried part has settled in every lane.
  // EMIT: the block computes and stores y; without it (pass 1 before the
  // predicted settle point of a chunk c >= 1, whose y pass 2 writes) only the
  // state is advanced.
  auto do_block = [&](auto emit_tag, int bb, const T (&dq)[kTok], const T (&xx)[kTok], const T (&zz)[kTok],
                      const T (&ll)[kTok], const T& dn, const T& ln, const Pair<T>& pb, const Pair<T>& pc)
                      __attribute__((always_inline)) {
    constexpr bool EMIT = decltype(emit_tag)::value;
    const auto ry = rsrc(yrow + (int64_t)bb * d_inner);
    // TR: delta and lam of the block's tokens and of the one after it (a
    // padding token's or a missing one's delta is 0), and C_t . B_t summed
    // over the 8 lanes of each token (lane 8 j holds token j's).
    float dtv[kTok + 1], lv[kTok + 1], cbl = 0.0f;
    if constexpr (TR) {
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        dtv[j] = bb + j < nt ? pro.dt(widen(dq[j])) : 0.0f;
        lv[j] = widen(ll[j]) + lam_add;
      }
      dtv[kTok] = t0 + bb + kTok < L ? pro.dt(widen(dn)) : 0.0f;
      lv[kTok] = widen(ln) + lam_add;
      if constexpr (EMIT) {
        cbl = pb.dot(pc);
        cbl += dpp_mov<0xB1>(cbl);        // lane ^ 1
        cbl += dpp_mov<0x4E>(cbl);        // lane ^ 2
        cbl += dpp_mov<0x141>(cbl);       // lane ^ 7 within 8 lanes
      }
    }
    float bsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      if constexpr (EMIT) Cv.load(crow + (int64_t)std::min(bb + j, nt - 1) * NSTATE);
      if constexpr (RMS) s_next = load_uniform(srow + std::min(bb + j + 1, nt - 1));
      // A padding token's delta reads 0; softplus would turn that into a
      // positive step, so it is forced back to 0 (a wave-uniform select).
      const float dts = SP ? pro.dt(raw_dt(dq[j])) : 0.0f;     // evaluated unconditionally: a select, no branch
      const float dt = TR ? dtv[j] : SP ? (bb + j < nt ? dts : 0.0f) : raw_dt(dq[j]);
      const float xv = pro.xin(widen(xx[j]));
      float dx = dt * xv, wn = 0.0f;
      if constexpr (TR) {
        wn = dtv[j + 1] * (1.0f - lv[j + 1]) * xv;        // w_{t+1}
        dx = fmaf(dx, lv[j], wn);                          // dt lam x + w_{t+1}
      }
      if constexpr (MODE != kWhole) bsum += dt;
      if constexpr (MODE == kLocal && !SP) negbits |= __float_as_uint(dt);
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dx * Bc[n]);
      // The next token's B row goes into the registers this token's row
      // held, while C . h and the epilogue run.
      Bc.load(brow + (int64_t)std::min(bb + j + 1, nt - 1) * NSTATE);
      if constexpr (EMIT) {
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < NSTATE; ++n) acc = fmaf(Cv[n], h[n], acc);
        if constexpr (TR)
          acc = fmaf(-wn, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cbl), 8 * j)), acc);
        finish(ry, bb, j, acc, xv, widen(zz[j]));
      }
      if constexpr (RMS) s_cur = s_next;
      // Keep each token's scalar B/C loads in its own token: hoisting them
      // across tokens would hold several rows in SGPRs at once and spill.
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == kLocal) {
      dacc += (double)bsum;
      aux.rec.after_block(bb + kTok, nt, b, c, h, dacc, d_inner, gbase, lo == lane, (uint32_t)lo * 4, sub_cur);
    }
    if constexpr (MODE == kFix) {
      fsum += bsum;
      // A bound on the part of the state pass 1 missed (exp2 of very
      // negative arguments is 0); sum delta counts from the chunk start.
      const float dm = fast_exp2(fix_a2 * fsum) * fix_h;
      float hm = 0.0f;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) hm = fmaxf(hm, fabsf(h[n]));
      // never before the point from which pass 1 wrote y
      const bool settled = can_exit && bb + kTok >= fix_from && dm <= hm * kSettled;    // false for NaN
      return __builtin_amdgcn_ballot_w64(!settled) == 0;
    }
    return false;
  };


  // Two register sets in turn: block i+1 is in flight while block i computes.
  T dA[kTok], xA[kTok], zA[kTok], lA[kTok], dnA, lnA;
  T dB[kTok], xB[kTok], zB[kTok], lB[kTok], dnB, lnB;
  Pair<T> pbA, pcA, pbB, pcB;
  load_block(0, dA, xA, zA, lA, dnA, lnA, pbA, pcA);
  __builtin_amdgcn_s_waitcnt(0);
  // Prefetches past the chunk's end are clamped to its last block (valid rows,
  // values unused), so every row offset below stays non-negative.
  const int last = (nt - 1) / kTok * kTok;
  const ProgressPrio prio(nt);
  // Pairs of blocks, one register set each, the next block's loads in
  // flight while a block computes.  Returns true when the chunk is done (or
  // pass 2 may stop after this pair), false when a state-only pass reaches
  // the point from which it must write y; `base` is then the next pair's
  // first token.
  int base = 0;
  auto pairs = [&](auto emit_tag) __attribute__((always_inline)) {
    constexpr bool EMIT = decltype(emit_tag)::value;
    for (; base < nt; base += 2 * kTok) {
      // The pair's first B row (and RMSNorm scale) is loaded here, not
      // carried over the loop's back edge: a row carried there is copied
      // into VGPRs, 16 of them for fp32 rows.
      Bc.load(brow + (int64_t)base * NSTATE);
      if constexpr (RMS) s_cur = load_uniform(srow + base);
      prio.set(base);
      load_block(std::min(base + kTok, last), dB, xB, zB, lB, dnB, lnB, pbB, pcB);
      const bool settled = do_block(emit_tag, base, dA, xA, zA, lA, dnA, lnA, pbA, pcA);
      if (base + kTok >= nt) return true;
      load_block(std::min(base + 2 * kTok, last), dA, xA, zA, lA, dnA, lnA, pbA, pcA);
      // pass 2 leaves at a pair's end (one exit per iteration keeps the
      // register allocation of the two blocks apart)
      if (do_block(emit_tag, base + kTok, dB, xB, zB, lB, dnB, lnB, pbB, pcB) || settled) return true;
      if constexpr (!EMIT) {
        // The carried-in part of the state has decayed by exp(A * sum delta)
        // since the chunk start, at most exp2(a2max * sum delta) for the
        // slowest state: once that is below 2^-24 in every lane, pass 2 can
        // stop here, so y from the next pair on is this pass's to write.
        if (__builtin_amdgcn_ballot_w64(!(dacc >= settle_sum)) == 0) {
          base += 2 * kTok;
          return false;
        }
      }
    }
    return true;
  };
  if constexpr (MODE == kLocal) {
    if (!emit && !pairs(std::false_type{})) {
      emit = true;
      emit_from = base;
    }
    if (emit && base < nt) pairs(std::true_type{});
  } else {
    pairs(std::true_type{});
  }
  if constexpr (MODE == kLocal) {
    if (lo == lane) aux.neg[(b * aux.chunks + c) * d_inner + d] = (negbits & 0x80000000u) ? 1 : 0;
    if (lane == 0) {
      prog[0] = emit ? emit_from : nt;
      prog[1] = 0;
    }
  }
  if constexpr (MODE == kFix) {
    if (lane == 0) prog[1] = std::min(base + 2 * kTok, nt);
  }
  if constexpr (MODE == kWhole) {
    if (aux.hT && lo == lane) {
      float* ho = aux.hT + (b * d_inner + d) * NSTATE;
#pragma unroll
      for (int n = 0; n < NSTATE; ++n) ho[n] = h[n];
    }
    // Conv history after the sequence: its last width-1 raw x (read back from
    // x, or from the history before it when the sequence is shorter).
    if constexpr (CONV) {
      if (pa.hist_out && lo == lane) {
        for (int j = 0; j < pa.width - 1; ++j) {
          const float v = pro.before(pa, pa.hist, x, b, L, d_inner, L - (pa.width - 1) + j, d);
          pa.hist_out[(b * (pa.width - 1) + j) * d_inner + d] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------ input RMSNorm
// RMSNorm of the scan's inputs, v / sqrt(mean v^2 + eps) * w per token, over
// the d_inner channels of the time step and over the 16 entries of each B and
// C row.  This pre-pass writes, in fp32 (nothing is rounded to the I/O
// dtype): s[row] = the time step's inverse root-mean-square (1 without a
// weight), and the normalised B and C rows (a null weight copies the row).
// The scan then reads delta * w[d] * s[t] and the fp32 rows.  One workgroup
// per token row (grid-stride over rows); the time step's sum of squares is
// reduced in-wave by shuffles and across the four waves through LDS, reading
// 16-byte vectors when a row's size allows.
template <class T>
__global__ __launch_bounds__(256) void k_rms_prep(const T* __restrict__ delta, const T* __restrict__ B,
                                                  const T* __restrict__ C, const float* __restrict__ w_dt,
                                                  const float* __restrict__ w_B, const float* __restrict__ w_C,
                                                  float eps, int64_t rows, int64_t d_inner, float* __restrict__ s_out,
                                                  float* __restrict__ B_out, float* __restrict__ C_out) {
  constexpr int V = 16 / sizeof(T);                  // elements per 16-byte vector
  __shared__ float part[4];
  const bool vec = d_inner % V == 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    if (w_dt) {
      const T* src = delta + row * d_inner;
      float ss = 0.0f;
      if (vec) {
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
      __syncthreads();                               // part[] of the previous row is consumed
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
      __syncthreads();
      if (threadIdx.x == 0)
        s_out[row] = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d_inner + eps);
    } else if (threadIdx.x == 0) {
      s_out[row] = 1.0f;
    }
    // B row on lanes 0-15, C row on lanes 16-31: one entry per lane
    if (threadIdx.x < 2 * NSTATE) {
      const int k = threadIdx.x / NSTATE, n = threadIdx.x % NSTATE;
      const float* w = k ? w_C : w_B;
      const float v = widen((k ? C : B)[row * NSTATE + n]);
      float q = v * v;
#pragma unroll
      for (int m = NSTATE / 2; m >= 1; m >>= 1) q += __shfl_xor(q, m, NSTATE);
      const float out = w ? v * (1.0f / sqrtf(q / (float)NSTATE + eps)) * w[n] : v;
      (k ? C_out : B_out)[row * NSTATE + n] = out;
    }
  }
}

// Copy (or zero) the state for an empty sequence: hT = h0, or 0 when h0 is
// null.  Grid-stride, so any size fits a capped grid.
__global__ __launch_bounds__(256) void k_copy_state(const float* __restrict__ src, float* __restrict__ dst,
                                                    int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
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
//
// The step is bound by memory latency as much as by bandwidth: each wave
// makes one access to each array.  So every load is issued first, with no
// branch among them, and the wave waits for memory once.  An optional array
// that is absent is read at a valid address of a required array of the same
// or larger size, and its value is replaced by the default with a
// wave-uniform select.
template <class T, bool CONV = false, bool SP = false, bool TR = false, bool RMS = false>
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
  const int64_t s = (uint32_t)sd / (uint32_t)d_inner;   // 32-bit: sd < n_seq * d_inner < 2^30
  const int64_t d = sd - s * d_inner;
  using RT = std::conditional_t<RMS, float, T>;

  float4 hv = reinterpret_cast<const float4*>(state)[g];
  const float4 av = reinterpret_cast<const float4*>(A)[d * 4 + q];
  const float xraw = widen(x[sd]);
  float dtr = widen(delta[sd]);
  const float zv = widen(z[sd]);
  const float Dd = D[d];
  // RMSNorm (prepared by k_rms_prep, one row per sequence): delta * w[d] *
  // s[seq], and the normalised fp32 B and C rows
  const RT* Bs;
  const RT* Cs;
  if constexpr (RMS) {
    Bs = pa.rms_B + s * NSTATE + 4 * q;
    Cs = pa.rms_C + s * NSTATE + 4 * q;
  } else {
    Bs = B + s * NSTATE + 4 * q;
    Cs = C + s * NSTATE + 4 * q;
  }
  float bq[4], cq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bq[k] = widen(Bs[k]);
    cq[k] = widen(Cs[k]);
  }
  // The prologue's and the trapezoidal form's inputs, as loaded (an absent
  // array read at a fallback address).
  const int hw = pa.width - 1;                  // history length (0..3)
  const bool use_hist = CONV && pa.hist && hw > 0;
  float tap[4] = {0.f, 0.f, 0.f, 0.f}, cb_raw = 0.f, hist_raw[3] = {0.f, 0.f, 0.f};
  float dtb_raw = 0.f, rw_raw = 1.f, rs_raw = 1.f, lam_raw = 0.f, xp_raw = 0.f;
  float bp[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (CONV) {
    // tap k of the caller's width-W filter goes to slot 4 - W + k (as in
    // Prologue::init); slots before the filter read tap 0 and are zeroed below
    const int W = pa.width;
    const float* wr = pa.conv_w + d * W;
#pragma unroll
    for (int m = 0; m < 4; ++m) tap[m] = wr[std::max(m + W - 4, 0)];
    cb_raw = opaque_global(pa.conv_b ? pa.conv_b : D)[d];
    // without a history the reads go to the state (more than 3 floats per
    // channel), and their values are dropped
    const auto* hp = opaque_global<float>(use_hist ? pa.hist : state);
#pragma unroll
    for (int j = 0; j < 3; ++j) hist_raw[j] = hp[(s * hw + std::max(std::min(j, hw - 1), 0)) * d_inner + d];
  }
  if constexpr (SP) dtb_raw = opaque_global(pa.dt_bias ? pa.dt_bias : D)[d];
  if constexpr (RMS) {
    rw_raw = opaque_global(pa.rms_w ? pa.rms_w : D)[d];
    rs_raw = pa.rms_s[s];
  }
  if constexpr (TR) {
    // lam and x_prev are [n_seq][d_inner] like x, B_prev [n_seq][16] like B
    lam_raw = widen(opaque_global(pa.lam ? static_cast<const T*>(pa.lam) : x)[sd]);
    xp_raw = widen(opaque_global(pa.x_prev ? static_cast<const T*>(pa.x_prev) : x)[sd]);
    const auto* Bq = opaque_global(pa.B_prev ? static_cast<const T*>(pa.B_prev) : B) + s * NSTATE + 4 * q;
#pragma unroll
    for (int k = 0; k < 4; ++k) bp[k] = widen(Bq[k]);
  }
  // Every load is in flight: wait for them together (values used only
  // under a branch would otherwise be loaded there, after this wait).
  keep(zv);
  keep(Dd);
  if constexpr (CONV) {
#pragma unroll
    for (int m = 0; m < 4; ++m) keep(tap[m]);
    keep(cb_raw);
#pragma unroll
    for (int j = 0; j < 3; ++j) keep(hist_raw[j]);
  }
  if constexpr (SP) keep(dtb_raw);
  if constexpr (RMS) {
    keep(rw_raw);
    keep(rs_raw);
  }
  if constexpr (TR) {
    keep(lam_raw);
    keep(xp_raw);
#pragma unroll
    for (int k = 0; k < 4; ++k) keep(bp[k]);
  }

  Prologue<CONV, SP> pro;
  float hist[3] = {0.f, 0.f, 0.f};              // oldest first: x[t-(width-1)] .. x[t-1]
  if constexpr (CONV) {
    const int W = pa.width;
    pro.w0 = W >= 4 ? tap[0] : 0.f;
    pro.w1 = W >= 3 ? tap[1] : 0.f;
    pro.w2 = W >= 2 ? tap[2] : 0.f;
    pro.w3 = tap[3];
    pro.cb = pa.conv_b ? cb_raw : 0.f;
#pragma unroll
    for (int j = 0; j < 3; ++j) hist[j] = use_hist && j < hw ? hist_raw[j] : 0.f;
    // x[t-1], x[t-2], x[t-3] out of the history, oldest first
    pro.h1 = hw == 3 ? hist[2] : hw == 2 ? hist[1] : hw == 1 ? hist[0] : 0.f;
    pro.h2 = hw == 3 ? hist[1] : hw == 2 ? hist[0] : 0.f;
    pro.h3 = hw == 3 ? hist[0] : 0.f;
  }
  if constexpr (SP) pro.dtb = pa.dt_bias ? dtb_raw : 0.f;
  if constexpr (RMS) dtr = dtr * (pa.rms_w ? rw_raw : 1.0f) * rs_raw;
  const float lam = TR && pa.lam ? lam_raw : 0.5f;
  const float xp = TR && pa.x_prev ? xp_raw : 0.f;

  const float xv = pro.xin(xraw);
  const float dt = pro.dt(dtr);
  float dx = dt * xv;
  if constexpr (TR) {
    // h = a (h + w B_prev) + v B with w = dt (1 - lam) x_prev, v = dt lam x
    const float wv = dt * (1.0f - lam) * xp;
    dx *= lam;
    if (pa.B_prev) {
      hv.x = fmaf(wv, bp[0], hv.x);
      hv.y = fmaf(wv, bp[1], hv.y);
      hv.z = fmaf(wv, bp[2], hv.z);
      hv.w = fmaf(wv, bp[3], hv.w);
    }
  }
  hv.x = fmaf(fast_exp2(dt * (av.x * kLog2e)), hv.x, dx * bq[0]);
  hv.y = fmaf(fast_exp2(dt * (av.y * kLog2e)), hv.y, dx * bq[1]);
  hv.z = fmaf(fast_exp2(dt * (av.z * kLog2e)), hv.z, dx * bq[2]);
  hv.w = fmaf(fast_exp2(dt * (av.w * kLog2e)), hv.w, dx * bq[3]);
  float part = cq[0] * hv.x;
  part = fmaf(cq[1], hv.y, part);
  part = fmaf(cq[2], hv.z, part);
  part = fmaf(cq[3], hv.w, part);
  part += __shfl_xor(part, 1, 4);
  part += __shfl_xor(part, 2, 4);
  if (active) {
    reinterpret_cast<float4*>(state)[g] = hv;
    if (q == 0) {
      store_io(y + sd, fmaf(Dd, xv, part) * silu(zv));
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

// Relative throughput of the backward's sweeps with `waves` waves launched on
// the 1024 SIMDs, measured on MI355X with the one-wave-per-64-channels
// kernels: one wave per SIMD issues at most every other cycle, a few more
// hide the load and exp latencies, and many more even out the tail across
// CUs.
double wave_efficiency(double waves) {
  static const double lw[] = {10, 11, 12, 13, 14, 15};
  static const double ef[] = {0.37, 0.53, 0.68, 0.91, 0.96, 1.0};
  const double l = std::log2(std::max(1.0, waves));
  if (l <= lw[0]) return ef[0] * waves / 1024.0;
  for (int i = 1; i < 6; ++i)
    if (l <= lw[i]) return ef[i - 1] + (ef[i] - ef[i - 1]) * (l - lw[i - 1]);
  return 1.0;
}

// Throughput of one SIMD running the forward scan with k resident waves,
// relative to four (measured on MI355X at batch 1 x 64K and batch 8 x 16K
// with the progress priority): one wave issues well under half the time, two
// reach about three quarters.  A SIMD holds at most four of these one-wave
// workgroups (a compute unit takes at most 16 workgroups), so a launch runs in
// rounds of 4096 waves.
constexpr int kResidentWaves = 4 * 4 * kCUs;
double simd_throughput(int k) {
  static const double t[] = {0.0, 0.45, 0.75, 0.92, 1.0};
  return t[std::min(std::max(k, 0), 4)];
}

// Time of a scan launch with `waves` waves of `tokens` tokens each, in units
// of a token step of one wave at full occupancy; a wave's setup (parameters,
// starting state, the first block's loads) costs about kWaveSetup steps.
constexpr double kWaveSetup = 24.0;
double scan_time(double waves, double tokens) {
  if (waves <= 0 || tokens <= 0) return 0.0;
  tokens += kWaveSetup;
  const double rounds = std::floor(waves / kResidentWaves);
  const double rest = waves - rounds * kResidentWaves;
  double t = rounds * 4.0 * tokens;                       // full rounds: 4 waves per SIMD
  if (rest > 0) {
    const int k = (int)std::ceil(rest / (4.0 * kCUs));    // waves per SIMD in the last round
    t += k * tokens / simd_throughput(k);
  }
  return t;
}

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Workgroups of 256 for a grid-stride pass over n elements (capped).
unsigned copy_grid(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20)); }

// The decode step runs four lanes per (sequence, channel) in a
// one-dimensional grid, which holds at most 2^32 work-items.
constexpr int64_t kMaxStepChannels = ((int64_t)1 << 30) - 64;

// Pieces of about L / n tokens: a multiple of kTok, n' = ceil(L / len) of them.
void split(int64_t L, int64_t n, int64_t* len, int* count) {
  const int64_t Lp = std::max<int64_t>(L, 1);
  if (L <= 0 || n <= 1) { *len = Lp; *count = 1; return; }
  int64_t l = (L + n - 1) / n;
  l = (l + kTok - 1) / kTok * kTok;
  *len = l;
  *count = (int)((L + l - 1) / l);
}

// Sub-chunk count: the granularity of the backward's sweeps, from their cost
// per channel-token (about 150 issue slots over the efficiency of their wave
// count, plus a chunk-local adjoint pass of about 115 on the (C-1)/C of the
// tokens that need a carry, run on segments that fill about 32 waves per
// SIMD).
int64_t choose_subs(int64_t batch, int64_t L, int64_t d_inner) {
  const int64_t groups = batch * ((d_inner + 63) / 64);
  if (L <= 0 || groups <= 0) return 1;
  int64_t best = 1;
  double best_cost = 1e300;
  for (int64_t C = 1; C <= 4096; C *= 2) {
    if (C > 1 && L / C < kMinChunk) break;
    int64_t len;
    int subs;
    split(L, C, &len, &subs);
    const int64_t want = (32 * 4 * kCUs) / (groups * std::max(1, subs - 1));
    const int64_t F = std::max<int64_t>(1, std::min<int64_t>(want, len / kMinChunk));
    double cost = 150.0 / wave_efficiency((double)groups * subs);
    if (subs > 1) cost += 115.0 * (double)(subs - 1) / subs / wave_efficiency((double)groups * (subs - 1) * F);
    if (cost < best_cost * 0.999) { best = subs; best_cost = cost; }
  }
  return best;
}

// Forward chunk count from the estimated time of pass 1 (every token, at the
// occupancy its wave count reaches) and pass 2 (about kFixTokens tokens of
// every chunk but the first: the carried-in state decays below fp32
// resolution within about 100 tokens at the configurations' decay rates, and
// a pass-2 token costs about 1.2 pass-1 tokens), plus a small fixed cost per
// launch (about 8 token steps).  At batch 1 x 64K this picks 32 chunks: one round of four waves per
// SIMD.
Plan choose_plan(int64_t batch, int64_t L, int64_t d_inner) {
  Plan p{1, std::max<int64_t>(L, 1), 1, std::max<int64_t>(L, 1)};
  if (t_force_chunks > 0) {
    split(L, std::min<int64_t>(t_force_chunks, std::max<int64_t>(L, 1)), &p.chunk_len, &p.chunks);
    p.sub_len = p.chunk_len;
    p.subs = p.chunks;
    return p;
  }
  const int64_t groups = batch * ((d_inner + 63) / 64);
  if (L <= 0 || groups <= 0) return p;
  split(L, choose_subs(batch, L, d_inner), &p.sub_len, &p.subs);
  constexpr double kFixTokens = 128.0, kLaunch = 8.0;
  double best = 1e300;
  for (int64_t C = 1; C <= 4096; C = C < 8 ? C + 1 : C * 2) {
    if (C > 1 && L / C < kMinChunk) break;
    int64_t len;
    int chunks;
    split(L, C, &len, &chunks);
    double t = scan_time((double)groups * chunks, (double)len);
    if (chunks > 1)
      t += 1.2 * scan_time((double)groups * (chunks - 1), std::min<double>((double)len, kFixTokens)) + 2 * kLaunch;
    if (t < best * 0.999) { best = t; p.chunks = chunks; p.chunk_len = len; }
  }
  return p;
}

WsLayout ws_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p) {
  (void)L;
  WsLayout w{};
  if (p.recorded()) {
    const size_t B = (size_t)batch, Dn = (size_t)d_inner, C = (size_t)p.chunks;
    w.tag = round_up(kTagWords * sizeof(int64_t));
    w.eS = round_up(B * C * NSTATE * Dn * sizeof(float));
    w.eL = round_up(B * C * Dn * sizeof(float));
    w.neg = round_up(B * C * Dn * sizeof(int32_t));
    w.from = round_up(B * C * (size_t)((d_inner + 63) / 64) * 2 * sizeof(int32_t));
    w.H = round_up(B * C * NSTATE * Dn * sizeof(float));
    if (p.subs > 1) {
      w.sS = round_up(B * (size_t)p.subs * NSTATE * Dn * sizeof(float));
      w.sL = round_up(B * (size_t)p.subs * Dn * sizeof(float));
    }
  }
  w.total = w.tag + w.eS + w.eL + w.neg + w.from + w.H + w.sS + w.sL;
  return w;
}

Tag make_tag(int64_t batch, int64_t L, int64_t d_inner, const Plan& p, int variant) {
  return Tag{{kTagMagic, batch, L, d_inner, p.chunks, p.chunk_len, p.sub_len, variant}};
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

template <class T, bool CONV, bool SP, bool TR, bool RMS, int MODE>
hipError_t launch_scan(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, void* y, const ScanAux& aux, const ProArgs& pa,
                       unsigned chunks, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)((aux.d_inner + 63) / 64), chunks, (unsigned)batch);
  hipLaunchKernelGGL((k_scan<T, CONV, SP, TR, RMS, MODE>), grid, dim3(64), 0, st, static_cast<const T*>(x),
                     static_cast<const T*>(delta), A, static_cast<const T*>(B), static_cast<const T*>(C), D,
                     static_cast<const T*>(z), static_cast<T*>(y), aux, pa);
  return hipGetLastError();
}

Records records_in(char* ws, const WsLayout& w, const Plan& p) {
  return Records{reinterpret_cast<float*>(ws + w.off_eS()), reinterpret_cast<float*>(ws + w.off_eL()),
                 p.subs > 1 ? reinterpret_cast<float*>(ws + w.off_sS()) : nullptr,
                 p.subs > 1 ? reinterpret_cast<float*>(ws + w.off_sL()) : nullptr, p.sub_len, p.chunks, p.subs};
}

template <class T, bool CONV, bool SP, bool TR, bool RMS>
jscan_status run_prefill(int64_t batch, int64_t L, int64_t d_inner, const void* x, const void* delta,
                         const float* A, const void* B, const void* C, const float* D, const void* z,
                         const float* h0, void* y, float* hT, char* ws, const Plan& p, const ProArgs& pa,
                         hipStream_t st) {
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  ScanAux aux{h0, hT, Records{}, nullptr, nullptr, nullptr, L, d_inner, p.chunk_len, p.chunks,
              (int)((d_inner + 63) / 64)};
  hipEvent_t eb = t_ev_before, ea = t_ev_after;
  t_ev_before = t_ev_after = nullptr;
  hipError_t e;
  if (eb && ea && (e = hipEventRecord(eb, st)) != hipSuccess) return hip_fail(e, "event record");
  if (!p.recorded()) {
    if ((e = launch_scan<T, CONV, SP, TR, RMS, kWhole>(x, delta, A, B, C, D, z, y, aux, pa, 1, batch, st)) !=
        hipSuccess)
      return hip_fail(e, "scan launch");
    if (eb && ea && (e = hipEventRecord(ea, st)) != hipSuccess) return hip_fail(e, "event record");
    return JSCAN_OK;
  }
  aux.rec = records_in(ws, w, p);
  aux.neg = reinterpret_cast<int32_t*>(ws + w.off_neg());
  aux.from = reinterpret_cast<int32_t*>(ws + w.off_from());
  float* H = reinterpret_cast<float*>(ws + w.off_H());
  aux.H = H;
  if ((e = launch_scan<T, CONV, SP, TR, RMS, kLocal>(x, delta, A, B, C, D, z, y, aux, pa, (unsigned)p.chunks, batch,
                                                st)) != hipSuccess)
    return hip_fail(e, "scan launch");
  if (eb && ea && (e = hipEventRecord(ea, st)) != hipSuccess) return hip_fail(e, "event record");
  const int variant = (CONV ? 1 : 0) | (SP ? 2 : 0) | (TR ? 4 : 0) | (RMS ? 8 : 0);
  dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL((k_combine<T>), g2, dim3(256), 0, st, A, aux.rec.eS, aux.rec.eL, H, hT, d_inner, p.chunks,
                     static_cast<const T*>(x), L, CONV ? pa : ProArgs{nullptr, nullptr, nullptr, nullptr, nullptr, 1},
                     reinterpret_cast<int64_t*>(ws), make_tag(batch, L, d_inner, p, variant));
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "combine launch");
  if (p.chunks > 1 &&
      (e = launch_scan<T, CONV, SP, TR, RMS, kFix>(x, delta, A, B, C, D, z, y, aux, pa, (unsigned)(p.chunks - 1), batch,
                                              st)) != hipSuccess)
    return hip_fail(e, "scan launch");
  return JSCAN_OK;
}

template <class T>
jscan_status records_t(int64_t batch, int64_t L, int64_t d_inner, const void* x, const void* delta, const float* A,
                       const void* B, const float* h0, char* rec, const Plan& p, hipStream_t st) {
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  const Records r = records_in(rec, w, p);
  hipError_t e;
  dim3 g1((unsigned)((d_inner + 255) / 256), (unsigned)p.chunks, (unsigned)batch);
  hipLaunchKernelGGL((k_chunk_state<T>), g1, dim3(256), 0, st, static_cast<const T*>(x),
                     static_cast<const T*>(delta), A, static_cast<const T*>(B), h0, r, L, d_inner, p.chunk_len);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "chunk-state launch");
  if (p.chunks > 1) {
    dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
    hipLaunchKernelGGL((k_combine<T>), g2, dim3(256), 0, st, A, r.eS, r.eL, reinterpret_cast<float*>(rec + w.off_H()),
                       nullptr, d_inner, p.chunks, static_cast<const T*>(x), L,
                       ProArgs{nullptr, nullptr, nullptr, nullptr, nullptr, 1}, nullptr, Tag{});
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "combine launch");
  }
  return JSCAN_OK;
}

jscan_status backward_records(jscan_io io, int64_t batch, int64_t L, int64_t d_inner, const void* x,
                              const void* delta, const float* A, const void* B, const float* h0, char* rec,
                              const char* saved, const Plan& p, hipStream_t st, SubRecords* out) {
  *out = SubRecords{};
  if (p.subs <= 1) return JSCAN_OK;
  if (!saved) {
    const jscan_status s = io == JSCAN_IO_BF16
                               ? records_t<uint16_t>(batch, L, d_inner, x, delta, A, B, h0, rec, p, st)
                               : records_t<float>(batch, L, d_inner, x, delta, A, B, h0, rec, p, st);
    if (s != JSCAN_OK) return s;
  }
  const char* base = saved ? saved : rec;
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  *out = SubRecords{reinterpret_cast<const float*>(base + w.off_sS()), reinterpret_cast<const float*>(base + w.off_sL()),
                    reinterpret_cast<const float*>(base + w.off_H())};
  return JSCAN_OK;
}

// Calls f(integral_constant<bool, CONV>, integral_constant<bool, SP>,
// integral_constant<bool, TR>, integral_constant<bool, RMS>) for the
// supported combinations (the trapezoidal form takes no convolution and no
// RMSNorm; callers reject those pairs first).
template <class F>
auto with_flags(bool conv, bool sp, bool tr, bool rms, F&& f) {
  using Y = std::true_type;
  using N = std::false_type;
  if (tr) return sp ? f(N{}, Y{}, Y{}, N{}) : f(N{}, N{}, Y{}, N{});
  auto pick = [&](auto r) {
    if (conv && sp) return f(Y{}, Y{}, N{}, r);
    if (conv) return f(Y{}, N{}, N{}, r);
    if (sp) return f(N{}, Y{}, N{}, r);
    return f(N{}, N{}, N{}, r);
  };
  return rms ? pick(Y{}) : pick(N{});
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

template <class T, bool CONV, bool SP, bool TR, bool RMS>
jscan_status run_step(int64_t n_seq, int64_t d_inner, float* state, const void* x, const void* delta,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      void* y, const ProArgs& pa, hipStream_t st) {
  const int64_t total = n_seq * d_inner * 4;
  hipLaunchKernelGGL((k_step<T, CONV, SP, TR, RMS>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, state,
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

// Bytes of the RMSNorm region for `rows` token rows: the time step's inverse
// root-mean-square per row, then the normalised B and C rows, all fp32.
size_t rms_bytes(int64_t rows) {
  return rows > 0 ? round_up((size_t)rows * 4) + 2 * round_up((size_t)rows * NSTATE * 4) : 0;
}

// Launches the RMSNorm pre-pass over `rows` token rows into `region`
// (rms_bytes(rows) bytes) and points pa's RMSNorm fields at the results.
jscan_status rms_prep(const jscan_prologue* pro, jscan_io io, int64_t rows, int64_t d_inner, const void* delta,
                      const void* B, const void* C, char* region, ProArgs* pa, hipStream_t st) {
  float* s_out = reinterpret_cast<float*>(region);
  float* B_out = reinterpret_cast<float*>(region + round_up((size_t)rows * 4));
  float* C_out = reinterpret_cast<float*>(region + round_up((size_t)rows * 4) + round_up((size_t)rows * NSTATE * 4));
  const unsigned grid = (unsigned)std::min<int64_t>(rows, 1 << 20);
  if (io == JSCAN_IO_BF16)
    hipLaunchKernelGGL((k_rms_prep<uint16_t>), dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(delta),
                       static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C), pro->rms_dt_weight,
                       pro->rms_B_weight, pro->rms_C_weight, pro->rms_eps, rows, d_inner, s_out, B_out, C_out);
  else
    hipLaunchKernelGGL((k_rms_prep<float>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(delta),
                       static_cast<const float*>(B), static_cast<const float*>(C), pro->rms_dt_weight,
                       pro->rms_B_weight, pro->rms_C_weight, pro->rms_eps, rows, d_inner, s_out, B_out, C_out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  pa->rms_s = s_out;
  pa->rms_w = pro->rms_dt_weight;
  pa->rms_B = B_out;
  pa->rms_C = C_out;
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

// ------------------------------------------------ allocation-free prefill
// jscan_prefill_noalloc keeps its chunk records in this array instead of a
// caller workspace: one copy per GPU, alive until the process ends.  Host code
// never passes `scratch` itself to a kernel (on the host the name is only a
// stand-in); it passes the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

jscan_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(JSCAN_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return JSCAN_OK;
}

jscan_status prefill_impl(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                          const void* x, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* h0, void* y, float* hT,
                          const jscan_prologue* pro, const jscan_trap* trap, void* workspace,
                          size_t workspace_bytes, void* stream, bool noalloc = false) {
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
  if (noalloc) {                 // no sub-chunk records for a backward: the forward's chunks only
    plan.subs = 1;
    plan.sub_len = std::max<int64_t>(L, 1);
  }
  const size_t rec_bytes = ws_layout(batch, L, d_inner, plan).total;
  const size_t need = rec_bytes + (has_rms(pro) ? rms_bytes(batch * L) : 0);
  if (noalloc && need > kScratchBytes)
    return fail(JSCAN_ERR_WORKSPACE, "jscan_prefill_noalloc: this problem needs " + std::to_string(need) +
                                         " bytes of scratch, more than its " + std::to_string(kScratchBytes));
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
        hipLaunchKernelGGL(k_copy_state, dim3(copy_grid(n)), dim3(256), 0, st, h0, hT, n);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "state copy launch");
      }
      if (pa.hist_out && pa.hist_out != pa.hist && pa.width > 1) {
        const int64_t n = batch * (pa.width - 1) * d_inner;
        hipLaunchKernelGGL(k_copy_state, dim3(copy_grid(n)), dim3(256), 0, st, pa.hist,
                           pa.hist_out, n);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "history copy launch");
      }
    }
    t_ev_before = t_ev_after = nullptr;
    return JSCAN_OK;
  }
  const bool conv = pa.conv_w != nullptr, sp = pro && pro->dt_softplus, tr = trap != nullptr, rms = has_rms(pro);
  if (noalloc && need > 0 && (s = scratch_address(&workspace)) != JSCAN_OK) return s;
  char* ws = static_cast<char*>(workspace);
  bool owned = false;
  if (!ws && need > 0) {
    if ((e = hipMallocAsync(reinterpret_cast<void**>(&ws), need, st)) != hipSuccess)
      return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }
  // RMSNorm: its per-token data go after the records, in the same workspace
  if (rms) s = rms_prep(pro, io, batch * L, d_inner, delta, B, C, ws + rec_bytes, &pa, st);
  if (s == JSCAN_OK)
    s = with_flags(conv, sp, tr, rms, [&](auto cv, auto spv, auto trv, auto rmv) {
      constexpr bool CV = decltype(cv)::value, SPV = decltype(spv)::value, TRV = decltype(trv)::value,
                     RMV = decltype(rmv)::value;
      return io == JSCAN_IO_BF16
                 ? run_prefill<uint16_t, CV, SPV, TRV, RMV>(batch, L, d_inner, x, delta, A, B, C, D, z, h0, y, hT,
                                                            ws, plan, pa, st)
                 : run_prefill<float, CV, SPV, TRV, RMV>(batch, L, d_inner, x, delta, A, B, C, D, z, h0, y, hT, ws,
                                                         plan, pa, st);
    });
  if (owned) {
    e = hipFreeAsync(ws, st);
    if (s == JSCAN_OK && e != hipSuccess) s = hip_fail(e, "hipFreeAsync(workspace)");
  }
  return s;
}

// workspace: the RMSNorm rows' region (rms_bytes(n_seq) bytes), or null to
// allocate it stream-ordered; unused without RMSNorm.
jscan_status step_impl(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io, float* state,
                       const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, void* y, const jscan_prologue* pro,
                       const jscan_trap* trap, void* stream, void* workspace = nullptr,
                       size_t workspace_bytes = 0) {
  t_last_error.clear();
  jscan_status s = check_common(d_state, io);
  if (s != JSCAN_OK) return s;
  int64_t t;
  // four lanes per (sequence, channel) in a one-dimensional grid of at most 2^32 work-items
  if (n_seq < 0 || d_inner < 0 || !mul_ok(n_seq, d_inner, &t) || t > kMaxStepChannels)
    return fail(JSCAN_ERR_SHAPE, "sizes must be >= 0 and n_seq * d_inner at most 2^30 - 64");
  if (n_seq == 0 || d_inner == 0) {                       // nothing to do; the prologue is still checked
    Range in[12], out[1];
    int n_in = 0, n_out = 0;
    ProArgs pa;
    jscan_status s2 = check_prologue(pro, n_seq, d_inner, &pa, in, &n_in, out, &n_out);
    return s2 != JSCAN_OK ? s2 : check_trap(trap, has_rms(pro), n_seq, 1, d_inner, 4, &pa, in, &n_in);
  }
  if (!state || !x || !delta || !A || !B || !C || !D || !z || !y)
    return fail(JSCAN_ERR_NULL, "every pointer is required");
  const void* ptrs[] = {state, x, delta, A, B, C, D, z, y, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const bool rms = has_rms(pro);
  const size_t need = rms ? rms_bytes(n_seq) : 0;
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)n_seq * (size_t)d_inner * es;
  const size_t rowb = (size_t)n_seq * NSTATE * es;
  const size_t stb = (size_t)n_seq * (size_t)d_inner * NSTATE * 4;
  Range in[20] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {B, rowb, "B"}, {C, rowb, "C"},
                  {A, (size_t)d_inner * NSTATE * 4, "A"}, {D, (size_t)d_inner * 4, "D"}};
  Range out[4] = {{y, tok, "y"}, {state, stb, "state"}};
  int n_in = 7, n_out = 2;
  if (workspace && need) out[n_out++] = Range{workspace, need, "workspace"};
  ProArgs pa;
  if ((s = check_prologue(pro, n_seq, d_inner, &pa, in, &n_in, out, &n_out)) != JSCAN_OK) return s;
  if ((s = check_trap(trap, rms, n_seq, 1, d_inner, es, &pa, in, &n_in)) != JSCAN_OK) return s;
  if ((s = check_ranges(in, n_in, out, n_out, pa.hist_out && pa.hist_out == pa.hist ? pa.hist : nullptr)) !=
      JSCAN_OK)
    return s;
  if (workspace && workspace_bytes < need)
    return fail(JSCAN_ERR_WORKSPACE, "workspace smaller than jscan_step_workspace_size()");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool conv = pa.conv_w != nullptr, sp = pro && pro->dt_softplus, tr = trap != nullptr;
  // RMSNorm: one row per sequence, in the caller's workspace or in
  // stream-ordered scratch
  char* rms_scratch = nullptr;
  if (rms) {
    char* region = static_cast<char*>(workspace);
    if (!region) {
      hipError_t e;
      if ((e = hipMallocAsync(reinterpret_cast<void**>(&rms_scratch), need, st)) != hipSuccess)
        return hip_fail(e, "hipMallocAsync(rmsnorm scratch)");
      region = rms_scratch;
    }
    s = rms_prep(pro, io, n_seq, d_inner, delta, B, C, region, &pa, st);
  }
  if (s == JSCAN_OK)
    s = with_flags(conv, sp, tr, rms, [&](auto cv, auto spv, auto trv, auto rmv) {
      constexpr bool CV = decltype(cv)::value, SPV = decltype(spv)::value, TRV = decltype(trv)::value,
                     RMV = decltype(rmv)::value;
      return io == JSCAN_IO_BF16
                 ? run_step<uint16_t, CV, SPV, TRV, RMV>(n_seq, d_inner, state, x, delta, A, B, C, D, z, y, pa, st)
                 : run_step<float, CV, SPV, TRV, RMV>(n_seq, d_inner, state, x, delta, A, B, C, D, z, y, pa, st);
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
    t_force_chunks = 0;
    return JSCAN_OK;
  }
  if (waves_per_group != 1 || chunks < 1 || chunks > kMaxChunks)
    return fail(JSCAN_ERR_UNSUPPORTED, "waves_per_group must be 1 and chunks in [1, 4096]");
  t_force_chunks = chunks;
  return JSCAN_OK;
}

jscan_status jscan_prefill_plan(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                int* waves_per_group, int* chunks) {
  if (d_state != NSTATE) return fail(JSCAN_ERR_UNSUPPORTED, "d_state must be 16");
  if (!sizes_ok(batch, L, d_inner)) return fail(JSCAN_ERR_SHAPE, "invalid sizes");
  const Plan p = choose_plan(batch, L, d_inner);
  if (waves_per_group) *waves_per_group = 1;
  if (chunks) *chunks = p.chunks;
  return JSCAN_OK;
}

jscan_status jscan_prefill_stats(const void* workspace, size_t workspace_bytes, int64_t batch, int64_t L,
                                 int64_t d_inner, double* stats, void* stream) {
  if (!workspace || !stats) return fail(JSCAN_ERR_NULL, "workspace and stats are required");
  if (!sizes_ok(batch, L, d_inner) || batch == 0 || L == 0 || d_inner == 0)
    return fail(JSCAN_ERR_SHAPE, "invalid sizes");
  const Plan p = choose_plan(batch, L, d_inner);
  stats[0] = stats[1] = 0.0;
  stats[2] = (double)p.chunks;
  if (p.chunks <= 1) return JSCAN_OK;
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  if (workspace_bytes < w.total) return fail(JSCAN_ERR_WORKSPACE, "workspace smaller than the plan's records");
  hipStream_t st = static_cast<hipStream_t>(stream);
  Tag tag;
  const int64_t groups = (d_inner + 63) / 64;
  std::vector<int32_t> prog((size_t)(batch * p.chunks * groups * 2));
  hipError_t e;
  if ((e = hipMemcpyAsync(&tag, workspace, sizeof(tag), hipMemcpyDeviceToHost, st)) != hipSuccess ||
      (e = hipMemcpyAsync(prog.data(), static_cast<const char*>(workspace) + w.off_from(),
                          prog.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st)) != hipSuccess ||
      (e = hipStreamSynchronize(st)) != hipSuccess)
    return hip_fail(e, "copy of the progress records");
  const Tag want = make_tag(batch, L, d_inner, p, 0);
  for (int i = 0; i < 6; ++i)     // magic, sizes and plan; any variant
    if (tag.w[i] != want.w[i]) return fail(JSCAN_ERR_WORKSPACE, "workspace holds no records of a prefill of these sizes");
  double total = 0, state_only = 0, rescanned = 0;
  for (int64_t b = 0; b < batch; ++b)
    for (int c = 1; c < p.chunks; ++c) {
      const double nt = (double)std::min<int64_t>(p.chunk_len, L - (int64_t)c * p.chunk_len);
      for (int64_t g = 0; g < groups; ++g) {
        const int32_t* r = &prog[(size_t)(((b * p.chunks + c) * groups + g) * 2)];
        total += nt;
        state_only += r[0];
        rescanned += r[1];
      }
    }
  stats[0] = state_only / total;
  stats[1] = rescanned / total;
  return JSCAN_OK;
}

size_t jscan_prefill_workspace_size(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                                    jscan_io io) {
  if (d_state != NSTATE || (io != JSCAN_IO_F32 && io != JSCAN_IO_BF16)) return 0;
  if (!sizes_ok(batch, L, d_inner)) return 0;
  // the records of the plan, and the RMSNorm region a fused call may need
  return ws_layout(batch, L, d_inner, choose_plan(batch, L, d_inner)).total + rms_bytes(batch * L);
}

jscan_status jscan_prefill(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                           const void* x, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* h0,
                           void* y, float* hT, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return prefill_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, y, hT, nullptr, nullptr,
                      workspace, workspace_bytes, stream);
}

jscan_status jscan_prefill_noalloc(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state, jscan_io io,
                                   const void* x, const void* delta, const float* A, const void* B,
                                   const void* C, const float* D, const void* z, const float* h0, void* y,
                                   float* hT, void* stream) {
  return prefill_impl(batch, L, d_inner, d_state, io, x, delta, A, B, C, D, z, h0, y, hT, nullptr, nullptr,
                      nullptr, 0, stream, true);
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

size_t jscan_step_workspace_size(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                 const jscan_prologue* prologue) {
  (void)d_inner;
  (void)io;
  if (d_state != NSTATE || n_seq <= 0 || n_seq > kMaxStepChannels || !has_rms(prologue)) return 0;
  return rms_bytes(n_seq);
}

jscan_status jscan_step_batch_fused_ws(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                                       float* state, const void* x, const void* delta, const float* A,
                                       const void* B, const void* C, const float* D, const void* z, void* y,
                                       const jscan_prologue* prologue, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return step_impl(n_seq, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, prologue, nullptr, stream,
                   workspace, workspace_bytes);
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
