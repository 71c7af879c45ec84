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
//   wave-uniform: they are read with scalar loads into SGPRs and fed to the
//   VALU as scalar operands, with no LDS traffic and no VGPRs.  For that the
//   rows are first widened to fp32 into the workspace by a small kernel.
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
#include <string>

#include "jscan.h"

namespace {

constexpr int NSTATE = 16;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kTok = 8;         // tokens per software-pipelined block
constexpr int kCUs = 256;       // MI355X compute units
constexpr int kWaveTarget = 2 * 4 * kCUs;   // two waves per SIMD
constexpr int64_t kMinChunk = 64;           // shortest chunk worth a carry

// ---------------------------------------------------------------- I/O types
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ void store_io(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);   // v_cvt_pk_bf16_f32: round to nearest even
}
__device__ __forceinline__ void store_io(float* p, float v) { *p = v; }

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// SiLU(z) = z / (1 + exp(-z)); v_exp_f32 and v_rcp_f32.  For z -> -inf the
// denominator is +inf and the result is -0, as in the definition.
__device__ __forceinline__ float silu(float zv) {
  return zv * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zv * kLog2e));
}

// ------------------------------------------------------- B/C row widening
// bc[r][0..15] = B[r][0..15], bc[r][16..31] = C[r][0..15], fp32.
template <class T>
__global__ __launch_bounds__(256) void k_widen_bc(const T* __restrict__ B, const T* __restrict__ C,
                                                  float* __restrict__ bc, int64_t rows) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * 32) return;
  const int64_t r = i >> 5;
  const int k = (int)(i & 31);
  bc[i] = k < NSTATE ? widen(B[r * NSTATE + k]) : widen(C[r * NSTATE + (k - NSTATE)]);
}

// ------------------------------------------------- chunk-local end states
// Load S consecutive floats from a wave-uniform address (scalar loads).
template <int S>
__device__ __forceinline__ void load_row(float (&v)[S], const float* __restrict__ p) {
  if constexpr (S % 4 == 0) {
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      const float4 w = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < S / 2; ++q) {
      const float2 w = reinterpret_cast<const float2*>(p)[q];
      v[2 * q] = w.x; v[2 * q + 1] = w.y;
    }
  }
}

template <int S>
__device__ __forceinline__ void copy_row(float (&dst)[S], const float (&src)[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) dst[s] = src[s];
}

// One lane per channel, all 16 states.  For chunk c (every chunk but the
// last) of sequence b: S[b][c][d][n] = state after the chunk when it starts
// from zero, dsum[b][c][d] = sum of delta over the chunk (accumulated in fp64).
template <class T>
__global__ __launch_bounds__(256) void k_chunk_state(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const float* __restrict__ bc, float* __restrict__ S, float* __restrict__ dsum,
    int64_t L, int64_t d_inner, int64_t chunk_len, int n_chunks) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const bool valid = d < d_inner;
  const int64_t dc = valid ? d : d_inner - 1;

  float a2[NSTATE], h[NSTATE];
  const float4* Ap = reinterpret_cast<const float4*>(A + dc * NSTATE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float4 v = Ap[q];
    a2[4 * q + 0] = v.x * kLog2e; a2[4 * q + 1] = v.y * kLog2e;
    a2[4 * q + 2] = v.z * kLog2e; a2[4 * q + 3] = v.w * kLog2e;
  }
#pragma unroll
  for (int n = 0; n < NSTATE; ++n) h[n] = 0.0f;
  double dacc = 0.0;

  const int64_t t0 = (int64_t)c * chunk_len;
  const int nt = (int)std::min<int64_t>(chunk_len, L - t0);   // >= 1 for every chunk
  const T* xp = x + (b * L + t0) * d_inner + dc;
  const T* dp = delta + (b * L + t0) * d_inner + dc;
  const float* bcrow = bc + (b * L + t0) * 32;

  auto token = [&](float dt, float xv, const float (&Bv)[NSTATE]) {
    const float dx = dt * xv;
    dacc += (double)dt;
#pragma unroll
    for (int n = 0; n < NSTATE; ++n) h[n] = fmaf(fast_exp2(dt * a2[n]), h[n], dx * Bv[n]);
  };

  T dr[kTok], xr[kTok];
#pragma unroll
  for (int j = 0; j < kTok; ++j) {
    const int64_t o = (int64_t)std::min(j, nt - 1) * d_inner;
    dr[j] = dp[o]; xr[j] = xp[o];
  }
  float Bc[NSTATE], Bn[NSTATE];
  load_row(Bc, bcrow);
  __builtin_amdgcn_s_waitcnt(0);
  int base = 0;
  for (; base + kTok <= nt; base += kTok) {
    T dn[kTok], xn[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {   // next block, clamped inside the chunk
      const int64_t o = (int64_t)std::min(base + kTok + j, nt - 1) * d_inner;
      dn[j] = dp[o]; xn[j] = xp[o];
    }
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      load_row(Bn, bcrow + (int64_t)std::min(base + j + 1, nt - 1) * 32);
      token(widen(dr[j]), widen(xr[j]), Bc);
      copy_row(Bc, Bn);
    }
#pragma unroll
    for (int j = 0; j < kTok; ++j) { dr[j] = dn[j]; xr[j] = xn[j]; }
  }
  for (; base < nt; ++base) {          // fewer than kTok tokens left
    const int64_t o = (int64_t)base * d_inner;
    load_row(Bc, bcrow + (int64_t)base * 32);
    token(widen(dp[o]), widen(xp[o]), Bc);
  }
  if (valid) {
    const int64_t slot = b * (n_chunks - 1) + c;
    float4* Sp = reinterpret_cast<float4*>(S + (slot * d_inner + d) * NSTATE);
#pragma unroll
    for (int q = 0; q < 4; ++q) Sp[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    dsum[slot * d_inner + d] = (float)dacc;
  }
}

// ------------------------------------------------------------ carry combine
// One lane per (b, d, n).  Folds the chunks' (P_c, S_c) pairs in sequence
// order, h <- P_c * h + S_c with P_c = exp2(A' * dsum_c), seeded with h0,
// and records the state each chunk starts from.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ A, const float* __restrict__ S,
                                                 const float* __restrict__ dsum, const float* __restrict__ h0,
                                                 float* __restrict__ hstart, int64_t d_inner, int n_chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t per_seq = d_inner * NSTATE;
  if (i >= per_seq) return;
  const int64_t d = i >> 4;
  const float a2 = A[i] * kLog2e;
  float h = h0 ? h0[b * per_seq + i] : 0.0f;
  for (int c = 0; c < n_chunks; ++c) {
    hstart[(b * n_chunks + c) * per_seq + i] = h;
    if (c + 1 < n_chunks) {
      const int64_t slot = b * (n_chunks - 1) + c;
      h = fmaf(fast_exp2(a2 * dsum[slot * d_inner + d]), h, S[slot * per_seq + i]);
    }
  }
}

// ----------------------------------------------------------------- main scan
struct ScanArgs {
  const void* x; const void* delta; const float* A; const float* bc; const float* D;
  const void* z; const float* hinit;   // h0 (single chunk) or hstart (chunked), may be null
  void* y; float* hT;
  int64_t L, d_inner, chunk_len;
  int n_chunks;
};

// Grid: (ceil(d_inner / 64), chunks, batch); block: K waves.  Wave g of a
// block owns states [g*16/K, (g+1)*16/K) of the block's 64 channels for the
// block's chunk of tokens.
template <class T, int K>
__global__ __launch_bounds__(64 * K) void k_scan(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const float* __restrict__ bc, const float* __restrict__ Dw, const T* __restrict__ z,
    const float* __restrict__ hinit, T* __restrict__ y, float* __restrict__ hT,
    int64_t L, int64_t d_inner, int64_t chunk_len, int n_chunks) {
  constexpr int S = NSTATE / K;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t d = (int64_t)blockIdx.x * 64 + lane;
  const int c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const bool valid = d < d_inner;
  const int64_t dc = valid ? d : d_inner - 1;
  const int n0 = g * S;

  float a2[S], h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) a2[s] = A[dc * NSTATE + n0 + s] * kLog2e;
  const float* hi = nullptr;
  if (n_chunks > 1) hi = hinit + ((b * n_chunks + c) * d_inner + dc) * NSTATE + n0;
  else if (hinit) hi = hinit + (b * d_inner + dc) * NSTATE + n0;
#pragma unroll
  for (int s = 0; s < S; ++s) h[s] = hi ? hi[s] : 0.0f;
  const float Dd = Dw[dc];

  const int64_t t0 = (int64_t)c * chunk_len;
  const int nt = (int)std::min<int64_t>(chunk_len, L - t0);   // >= 1 for every chunk
  const int64_t off0 = (b * L + t0) * d_inner + dc;
  const T* xp = x + off0;
  const T* dp = delta + off0;
  const T* zp = z + off0;
  T* yp = y + off0;
  const float* bcrow = bc + (b * L + t0) * 32;

  __shared__ float red[K > 1 ? K : 1][kTok][64];

  // State update for one token; returns this wave's share of sum_n C*h.
  auto token = [&](float dt, float xv, const float (&Bv)[S], const float (&Cv)[S]) {
    const float dx = dt * xv;
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      h[s] = fmaf(fast_exp2(dt * a2[s]), h[s], dx * Bv[s]);
      acc = fmaf(Cv[s], h[s], acc);
    }
    return acc;
  };
  // Lanes past d_inner run on the clamped channel d_inner - 1 with exactly the
  // same inputs and arithmetic as that channel's own lane, so their store
  // writes the identical value to the identical address; storing
  // unconditionally keeps the token loop free of branches.
  auto finish = [&](int64_t o, float acc, float xv, float zv) {
    store_io(yp + o, fmaf(Dd, xv, acc) * silu(zv));
  };
  // K > 1: add the K partial sums of tokens [base, base+count) through LDS;
  // wave g finishes the tokens j with j % K == g.
  auto reduce_block = [&](int base, const float (&part)[kTok], int count) {
#pragma unroll
    for (int j = 0; j < kTok; ++j) red[g][j][lane] = part[j];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTok / K; ++i) {
      const int j = i * K + g;
      if (j < count) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < K; ++w) acc += red[w][j][lane];
        const int64_t o = (int64_t)(base + j) * d_inner;
        finish(o, acc, widen(xp[o]), widen(zp[o]));
      }
    }
    __syncthreads();
  };

  T dr[kTok], xr[kTok], zr[kTok];
#pragma unroll
  for (int j = 0; j < kTok; ++j) {
    const int64_t o = (int64_t)std::min(j, nt - 1) * d_inner;
    dr[j] = dp[o]; xr[j] = xp[o];
    if constexpr (K == 1) zr[j] = zp[o];
  }
  float Bc[S], Cc[S], Bn[S], Cn[S];
  load_row(Bc, bcrow + n0);
  load_row(Cc, bcrow + NSTATE + n0);
  __builtin_amdgcn_s_waitcnt(0);

  int base = 0;
  for (; base + kTok <= nt; base += kTok) {
    T dn[kTok], xn[kTok], zn[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {   // next block, clamped inside the chunk
      const int64_t o = (int64_t)std::min(base + kTok + j, nt - 1) * d_inner;
      dn[j] = dp[o]; xn[j] = xp[o];
      if constexpr (K == 1) zn[j] = zp[o];
    }
    float part[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const float* nrow = bcrow + (int64_t)std::min(base + j + 1, nt - 1) * 32;
      load_row(Bn, nrow + n0);
      load_row(Cn, nrow + NSTATE + n0);
      const float xv = widen(xr[j]);
      const float acc = token(widen(dr[j]), xv, Bc, Cc);
      if constexpr (K == 1) finish((int64_t)(base + j) * d_inner, acc, xv, widen(zr[j]));
      else part[j] = acc;
      copy_row(Bc, Bn);
      copy_row(Cc, Cn);
    }
    if constexpr (K > 1) reduce_block(base, part, kTok);
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      dr[j] = dn[j]; xr[j] = xn[j];
      if constexpr (K == 1) zr[j] = zn[j];
    }
  }
  if (base < nt) {                     // fewer than kTok tokens left
    float part[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      part[j] = 0.0f;
      if (base + j < nt) {
        const int64_t o = (int64_t)(base + j) * d_inner;
        const float* row = bcrow + (int64_t)(base + j) * 32;
        load_row(Bc, row + n0);
        load_row(Cc, row + NSTATE + n0);
        const float xv = widen(xp[o]);
        const float acc = token(widen(dp[o]), xv, Bc, Cc);
        if constexpr (K == 1) finish(o, acc, xv, widen(zp[o]));
        else part[j] = acc;
      }
    }
    if constexpr (K > 1) reduce_block(base, part, nt - base);
  }
  if (hT && c == n_chunks - 1 && valid) {
    float* ho = hT + (b * d_inner + d) * NSTATE + n0;
#pragma unroll
    for (int s = 0; s < S; ++s) ho[s] = h[s];
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
template <class T>
__global__ __launch_bounds__(256) void k_step(float* __restrict__ state, const T* __restrict__ x,
                                              const T* __restrict__ delta, const float* __restrict__ A,
                                              const T* __restrict__ B, const T* __restrict__ C,
                                              const float* __restrict__ D, const T* __restrict__ z,
                                              T* __restrict__ y, int64_t n_seq, int64_t d_inner) {
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
  const float dt = widen(delta[sd]);
  const float xv = widen(x[sd]);
  const T* Bs = B + s * NSTATE + 4 * q;
  const T* Cs = C + s * NSTATE + 4 * q;
  const float dx = dt * xv;
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
    if (q == 0) store_io(y + sd, fmaf(D[d], xv, part) * silu(widen(z[sd])));
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

struct Range { const void* p; size_t bytes; const char* name; };

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Plan { int K; int chunks; int64_t chunk_len; };

// Pick the state split K and the chunk count for these sizes.  The model
// counts VALU issue slots per channel-token: the rescan costs about 145 + 4K
// (16 x (mul, exp at quarter rate, mul, fma, fma) plus the epilogue and the
// K-fold replication of the per-token loads), the chunk-local pass about 115
// on the (C-1)/C of the tokens that need a carry.  Candidates must give at
// least two waves per SIMD and one workgroup per CU where the sizes allow.
Plan choose_plan(int64_t batch, int64_t L, int64_t d_inner) {
  if (t_force_K > 0 && t_force_chunks > 0) {
    const int64_t C = std::max<int64_t>(1, std::min<int64_t>(t_force_chunks, L));
    const int64_t len = L > 0 ? (L + C - 1) / C : 1;
    return Plan{t_force_K, L > 0 ? (int)((L + len - 1) / len) : 1, len};
  }
  if (L <= 0) return Plan{1, 1, 1};
  const int64_t groups = batch * ((d_inner + 63) / 64);
  Plan best{1, 1, L};
  double best_cost = 1e300;
  bool best_fills = false;
  const int64_t max_chunks = std::max<int64_t>(1, L / kMinChunk);
  for (int K : {1, 2, 4, 8}) {
    for (int64_t C = 1; C <= 4096; C *= 2) {
      if (C > max_chunks && C > 1) break;
      const int64_t waves = groups * K * C;
      const int64_t wgs = groups * C;
      const bool fills = waves >= kWaveTarget && wgs >= kCUs;
      const double cost = (145.0 + 4.0 * K) + 115.0 * (double)(C - 1) / (double)C;
      // Prefer plans that fill the chip; among those the cheapest; if none
      // fills it, the one with the most waves (then the cheapest).
      bool better;
      if (fills != best_fills) better = fills;
      else if (fills) better = cost < best_cost;
      else {
        const int64_t bw = groups * best.K * best.chunks;
        better = waves > bw || (waves == bw && cost < best_cost);
      }
      if (better) {
        const int64_t len = (L + C - 1) / C;
        best = Plan{K, (int)((L + len - 1) / len), len};
        best_cost = cost;
        best_fills = fills;
      }
    }
  }
  return best;
}

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout { size_t bc, S, dsum, hstart, total; };

WsLayout ws_layout(int64_t batch, int64_t L, int64_t d_inner, const Plan& p) {
  WsLayout w{};
  w.bc = round_up((size_t)batch * (size_t)L * 32 * sizeof(float));
  if (p.chunks > 1) {
    w.S = round_up((size_t)batch * (size_t)(p.chunks - 1) * (size_t)d_inner * NSTATE * sizeof(float));
    w.dsum = round_up((size_t)batch * (size_t)(p.chunks - 1) * (size_t)d_inner * sizeof(float));
    w.hstart = round_up((size_t)batch * (size_t)p.chunks * (size_t)d_inner * NSTATE * sizeof(float));
  }
  w.total = w.bc + w.S + w.dsum + w.hstart;
  return w;
}

bool sizes_ok(int64_t batch, int64_t L, int64_t d_inner) {
  int64_t t;
  if (batch < 0 || L < 0 || d_inner < 0) return false;
  if (!mul_ok(batch, L, &t) || !mul_ok(t, d_inner, &t) || !mul_ok(t, 8, &t)) return false;
  if (!mul_ok(batch, d_inner, &t) || !mul_ok(t, NSTATE * 8, &t)) return false;
  if (!mul_ok(batch, L, &t) || !mul_ok(t, 32 * 8, &t)) return false;
  return L <= INT32_MAX && batch <= 65535;
}

template <class T, int K>
hipError_t launch_scan(const ScanArgs& a, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)((a.d_inner + 63) / 64), (unsigned)a.n_chunks, (unsigned)batch);
  hipLaunchKernelGGL((k_scan<T, K>), grid, dim3(64 * K), 0, st, static_cast<const T*>(a.x),
                     static_cast<const T*>(a.delta), a.A, a.bc, a.D, static_cast<const T*>(a.z), a.hinit,
                     static_cast<T*>(a.y), a.hT, a.L, a.d_inner, a.chunk_len, a.n_chunks);
  return hipGetLastError();
}

template <class T>
hipError_t launch_scan_k(int K, const ScanArgs& a, int64_t batch, hipStream_t st) {
  switch (K) {
    case 1: return launch_scan<T, 1>(a, batch, st);
    case 2: return launch_scan<T, 2>(a, batch, st);
    case 4: return launch_scan<T, 4>(a, batch, st);
    default: return launch_scan<T, 8>(a, batch, st);
  }
}

template <class T>
jscan_status run_prefill(int64_t batch, int64_t L, int64_t d_inner, const void* x, const void* delta,
                         const float* A, const void* B, const void* C, const float* D, const void* z,
                         const float* h0, void* y, float* hT, char* ws, const Plan& p,
                         hipStream_t st) {
  const WsLayout w = ws_layout(batch, L, d_inner, p);
  float* bc = reinterpret_cast<float*>(ws);
  float* S = reinterpret_cast<float*>(ws + w.bc);
  float* dsum = reinterpret_cast<float*>(ws + w.bc + w.S);
  float* hstart = reinterpret_cast<float*>(ws + w.bc + w.S + w.dsum);
  hipError_t e;

  const int64_t rows = batch * L;
  hipLaunchKernelGGL((k_widen_bc<T>), dim3((unsigned)((rows * 32 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const T*>(B), static_cast<const T*>(C), bc, rows);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "widen B/C launch");

  if (p.chunks > 1) {
    dim3 g1((unsigned)((d_inner + 255) / 256), (unsigned)(p.chunks - 1), (unsigned)batch);
    hipLaunchKernelGGL((k_chunk_state<T>), g1, dim3(256), 0, st, static_cast<const T*>(x),
                       static_cast<const T*>(delta), A, bc, S, dsum, L, d_inner, p.chunk_len, p.chunks);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "chunk-state launch");
    dim3 g2((unsigned)((d_inner * NSTATE + 255) / 256), (unsigned)batch);
    hipLaunchKernelGGL(k_combine, g2, dim3(256), 0, st, A, S, dsum, h0, hstart, d_inner, p.chunks);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "combine launch");
  }
  ScanArgs a{x, delta, A, bc, D, z, p.chunks > 1 ? hstart : h0, y, hT, L, d_inner, p.chunk_len, p.chunks};
  hipEvent_t eb = t_ev_before, ea = t_ev_after;
  t_ev_before = t_ev_after = nullptr;
  if (eb && ea && (e = hipEventRecord(eb, st)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = launch_scan_k<T>(p.K, a, batch, st)) != hipSuccess) return hip_fail(e, "scan launch");
  if (eb && ea && (e = hipEventRecord(ea, st)) != hipSuccess) return hip_fail(e, "event record");
  return JSCAN_OK;
}

jscan_status check_common(int64_t d_state, jscan_io io) {
  if (io != JSCAN_IO_F32 && io != JSCAN_IO_BF16) return fail(JSCAN_ERR_UNSUPPORTED, "io must be JSCAN_IO_F32 or JSCAN_IO_BF16");
  if (d_state != NSTATE) return fail(JSCAN_ERR_UNSUPPORTED, "d_state must be 16");
  return JSCAN_OK;
}

// Every output against every input and every other output.  An output may be
// the very same buffer as one input (`same_ok`, e.g. an in-place state carry).
jscan_status check_ranges(const Range* in, int n_in, const Range* out, int n_out,
                          const void* same_ok = nullptr) {
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

template <class T>
jscan_status run_step(int64_t n_seq, int64_t d_inner, float* state, const void* x, const void* delta,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      void* y, hipStream_t st) {
  const int64_t total = n_seq * d_inner * 4;
  hipLaunchKernelGGL((k_step<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, state,
                     static_cast<const T*>(x), static_cast<const T*>(delta), A, static_cast<const T*>(B),
                     static_cast<const T*>(C), D, static_cast<const T*>(z), static_cast<T*>(y), n_seq,
                     d_inner);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "step launch");
  return JSCAN_OK;
}

}  // namespace

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
  const Plan plan = choose_plan(batch, L, d_inner);
  const size_t need = ws_layout(batch, L, d_inner, plan).total;
  const Range in[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {B, rowb, "B"}, {C, rowb, "C"},
                      {A, (size_t)d_inner * NSTATE * 4, "A"}, {D, (size_t)d_inner * 4, "D"},
                      {h0, stb, "h0"}};
  const Range out[] = {{y, tok, "y"}, {hT, stb, "hT"}, {workspace, workspace ? need : 0, "workspace"}};
  if ((s = check_ranges(in, 8, out, 3, hT == h0 ? h0 : nullptr)) != JSCAN_OK) return s;
  if (workspace && workspace_bytes < need)
    return fail(JSCAN_ERR_WORKSPACE, "workspace smaller than jscan_prefill_workspace_size()");

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!work) {
    // Nothing to scan.  With L == 0 the final state is the initial state.
    if (hT && hT != h0 && L == 0 && batch > 0 && d_inner > 0) {
      const int64_t n = batch * d_inner * NSTATE;
      hipLaunchKernelGGL(k_copy_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, h0, hT, n);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "state copy launch");
    }
    t_ev_before = t_ev_after = nullptr;
    return JSCAN_OK;
  }
  char* ws = static_cast<char*>(workspace);
  bool owned = false;
  if (!ws) {
    if ((e = hipMallocAsync(reinterpret_cast<void**>(&ws), need, st)) != hipSuccess)
      return hip_fail(e, "hipMallocAsync(workspace)");
    owned = true;
  }
  s = io == JSCAN_IO_BF16
          ? run_prefill<uint16_t>(batch, L, d_inner, x, delta, A, B, C, D, z, h0, y, hT, ws, plan, st)
          : run_prefill<float>(batch, L, d_inner, x, delta, A, B, C, D, z, h0, y, hT, ws, plan, st);
  if (owned) {
    e = hipFreeAsync(ws, st);
    if (s == JSCAN_OK && e != hipSuccess) return hip_fail(e, "hipFreeAsync(workspace)");
  }
  return s;
}

jscan_status jscan_step_batch(int64_t n_seq, int64_t d_inner, int64_t d_state, jscan_io io,
                              float* state, const void* x, const void* delta, const float* A,
                              const void* B, const void* C, const float* D, const void* z,
                              void* y, void* stream) {
  t_last_error.clear();
  jscan_status s = check_common(d_state, io);
  if (s != JSCAN_OK) return s;
  int64_t t;
  if (n_seq < 0 || d_inner < 0 || !mul_ok(n_seq, d_inner, &t) || !mul_ok(t, NSTATE * 16, &t) ||
      t / (NSTATE * 16) > ((int64_t)1 << 37))
    return fail(JSCAN_ERR_SHAPE, "sizes must be >= 0 and fit 64-bit byte counts");
  if (n_seq == 0 || d_inner == 0) return JSCAN_OK;
  if (!state || !x || !delta || !A || !B || !C || !D || !z || !y)
    return fail(JSCAN_ERR_NULL, "every pointer is required");
  const void* ptrs[] = {state, x, delta, A, B, C, D, z, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(JSCAN_ERR_ALIGN, "every pointer must be 16-byte aligned");
  const size_t es = io == JSCAN_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)n_seq * (size_t)d_inner * es;
  const size_t rowb = (size_t)n_seq * NSTATE * es;
  const size_t stb = (size_t)n_seq * (size_t)d_inner * NSTATE * 4;
  const Range in[] = {{x, tok, "x"}, {delta, tok, "delta"}, {z, tok, "z"}, {B, rowb, "B"}, {C, rowb, "C"},
                      {A, (size_t)d_inner * NSTATE * 4, "A"}, {D, (size_t)d_inner * 4, "D"}};
  const Range out[] = {{y, tok, "y"}, {state, stb, "state"}};
  if ((s = check_ranges(in, 7, out, 2)) != JSCAN_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return io == JSCAN_IO_BF16 ? run_step<uint16_t>(n_seq, d_inner, state, x, delta, A, B, C, D, z, y, st)
                             : run_step<float>(n_seq, d_inner, state, x, delta, A, B, C, D, z, y, st);
}

jscan_status jscan_step(int64_t d_inner, int64_t d_state, jscan_io io, float* state, const void* x,
                        const void* delta, const float* A, const void* B, const void* C, const float* D,
                        const void* z, void* y, void* stream) {
  return jscan_step_batch(1, d_inner, d_state, io, state, x, delta, A, B, C, D, z, y, stream);
}

}  // extern "C"
