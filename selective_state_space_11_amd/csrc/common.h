// Device helpers shared by the forward and backward scan kernels of libjscan
// (gfx950): I/O widening and rounding, the fast transcendental forms, the
// optional input prologue, scalar-loaded B/C rows and raw buffer accesses.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace jscan_detail {

constexpr int NSTATE = 16;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kTok = 8;         // tokens per software-pipelined block
constexpr int kCUs = 256;       // MI355X compute units
constexpr int64_t kMinChunk = 64;           // shortest chunk worth a carry
constexpr int kMaxChunks = 4096;            // most chunks a forced plan may ask for

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

// softplus(v) = log(1 + exp(v)), through v_exp_f32 / v_log_f32 (base 2).  For
// v > 15 it equals v to fp32 precision; for tiny exp(v) log(1 + e) ~ e - e^2/2.
// Both candidates are evaluated before the selects: a select with v_log on
// one side would otherwise become a divergent branch, and the basic blocks it
// makes let the compiler pull the softplus and B-row loads of a whole token
// block ahead of the state updates (rows piling up in SGPRs).
__device__ __forceinline__ float softplus(float v) {
  const float e = fast_exp2(v * kLog2e);
  const float big = __builtin_amdgcn_logf(1.0f + e) * 0.69314718055994531f;
  const float small = e - 0.5f * e * e;
  const float r = e < 1.0e-3f ? small : big;
  return v > 15.0f ? v : r;
}

// Optional input prologue of a Mamba layer, applied per token as x and delta
// are loaded:
//   x  -> SiLU(conv_b + sum_k w[k] * x[t - (width - 1) + k])   (causal depthwise conv)
//   dt -> softplus(dt + dt_bias)
// The convolution keeps the last three raw x of its channel in registers;
// taps are right-aligned in a 4-tap window with the missing ones zero, which
// adds exact zeros.
struct ProArgs {
  const float* conv_w;      // [d_inner][width], or null: no convolution
  const float* conv_b;      // [d_inner], or null
  const float* hist;        // [batch][width-1][d_inner] history before the sequence, or null (zeros)
  float* hist_out;          // [batch][width-1][d_inner] history after it, or null
  const float* dt_bias;     // [d_inner], or null
  int width;
  // Exponential-trapezoidal recurrence (I/O dtype arrays): the weight lam_t
  // [nseq][L][d_inner] (null: 1/2), and x and the B row of the token before
  // the first, [nseq][d_inner] and [nseq][16] (null: zero).
  const void* lam = nullptr;
  const void* x_prev = nullptr;
  const void* B_prev = nullptr;
  // RMSNorm of the inputs, prepared per token by k_rms_prep in fp32: the
  // inverse root-mean-square of the time step over its channels [nseq][L]
  // (1 when the time step is not normalised), the time step's weight per
  // channel [d_inner] (null: 1), and the normalised B and C rows
  // [nseq][L][16].  The scan reads delta * w[d] * s[t] and these rows.
  const float* rms_s = nullptr;
  const float* rms_w = nullptr;
  const float* rms_B = nullptr;
  const float* rms_C = nullptr;
};

template <bool CONV, bool SP>
struct Prologue {
  float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, cb = 0.f, dtb = 0.f;
  float h1 = 0.f, h2 = 0.f, h3 = 0.f;       // raw x of tokens t-1, t-2, t-3
  __device__ __forceinline__ void init(const ProArgs& p, int64_t d) {
    if constexpr (CONV) {
      // tap k of the caller's width-W filter goes to slot 4 - W + k
      const float* wr = p.conv_w + d * p.width;
      const int off = 4 - p.width;
      w3 = wr[p.width - 1];
      w2 = off <= 2 ? wr[2 - off] : 0.f;
      w1 = off <= 1 ? wr[1 - off] : 0.f;
      w0 = off <= 0 ? wr[0] : 0.f;
      cb = p.conv_b ? p.conv_b[d] : 0.f;
    }
    if constexpr (SP) dtb = p.dt_bias ? p.dt_bias[d] : 0.f;
  }
  // Raw x before token t0 of sequence b: from x itself, or from the history
  // given for the sequence start (hist, or zeros).
  template <class T>
  __device__ __forceinline__ float before(const ProArgs& p, const float* hist, const T* x, int64_t b, int64_t L,
                                          int64_t d_inner, int64_t pos, int64_t d) const {
    if (pos >= 0) return widen(x[(b * L + pos) * d_inner + d]);
    const int64_t j = (p.width - 1) + pos;
    return (hist && j >= 0) ? hist[(b * (p.width - 1) + j) * d_inner + d] : 0.f;
  }
  template <class T>
  __device__ __forceinline__ void start(const ProArgs& p, const float* hist, const T* x, int64_t b, int64_t L,
                                        int64_t d_inner, int64_t t0, int64_t d) {
    if constexpr (CONV) {
      h1 = before(p, hist, x, b, L, d_inner, t0 - 1, d);
      h2 = before(p, hist, x, b, L, d_inner, t0 - 2, d);
      h3 = before(p, hist, x, b, L, d_inner, t0 - 3, d);
    }
  }
  __device__ __forceinline__ float xin(float xv) {
    if constexpr (CONV) {
      const float acc = fmaf(w3, xv, fmaf(w2, h1, fmaf(w1, h2, fmaf(w0, h3, cb))));
      h3 = h2; h2 = h1; h1 = xv;
      return silu(acc);
    } else {
      return xv;
    }
  }
  __device__ __forceinline__ float dt(float dv) const {
    if constexpr (SP) return softplus(dv + dtb);
    else return dv;
  }
};

// A wave-uniform address as a pointer into the constant address space: the
// address is taken from the first lane (it is the same in every lane), and
// loads through it are scalar (s_load into SGPRs).  Without this the
// compiler sometimes cannot prove a row address uniform and loads the row
// into VGPRs with a vector load, whose wait then also waits for every
// prefetch issued before it.  The rows read this way (B and C) are inputs
// that no kernel writes.
template <class V, class T>
__device__ __forceinline__ const __attribute__((address_space(4))) V* uniform_ptr(const T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                     (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return (const __attribute__((address_space(4))) V*)(uintptr_t)u;
}

// A wave-uniform pointer the compiler cannot see through: it can then no
// longer tie a load through it to the condition that chose it (and so place
// the load behind a branch), nor merge it with an earlier load of the same
// address.
template <class T>
__device__ __forceinline__ const T* opaque_ptr(const T* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// The same for a pointer into global memory, kept in the global address
// space so that loads through it stay global (not flat) loads.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* opaque_global(const T* p) {
  auto g = (const __attribute__((address_space(1))) T*)p;
  asm volatile("" : "+s"(g));
  return g;
}

// Marks v as used here: the load that produced it is then issued and waited
// for before this point, not moved behind a later branch that is the only
// other place its value is used.
__device__ __forceinline__ void keep(float v) { asm volatile("" ::"v"(v)); }

// Four dwords as a plain vector type (HIP's uint4 cannot be copied out of the
// constant address space).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Load S consecutive floats from a wave-uniform address (scalar loads).
template <int S>
__device__ __forceinline__ void load_row(float (&v)[S], const float* __restrict__ p) {
  if constexpr (S % 4 == 0) {
    const auto* q4 = uniform_ptr<u32x4>(p);
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      const u32x4 w = q4[q];
      v[4 * q] = __uint_as_float(w.x); v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z); v[4 * q + 3] = __uint_as_float(w.w);
    }
  } else {
    const auto* q1 = uniform_ptr<uint32_t>(p);
#pragma unroll
    for (int q = 0; q < S; ++q) v[q] = __uint_as_float(q1[q]);
  }
}

template <int S>
__device__ __forceinline__ void copy_row(float (&dst)[S], const float (&src)[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) dst[s] = src[s];
}

// S consecutive values of a B or C row, read with scalar loads from a
// wave-uniform address and kept in SGPRs in the I/O format.  bf16 pairs stay
// packed (S/2 dwords) and are widened when used (a scalar shift or mask).
template <class T, int S> struct Row;
template <int S> struct Row<uint16_t, S> {
  static_assert(S % 2 == 0, "bf16 rows are read in pairs");
  uint32_t w[S / 2];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p) {
    if constexpr (S % 8 == 0) {
      const auto* q4 = uniform_ptr<u32x4>(p);
#pragma unroll
      for (int q = 0; q < S / 8; ++q) {
        const u32x4 v = q4[q];
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    } else {
      const auto* q1 = uniform_ptr<uint32_t>(p);
#pragma unroll
      for (int q = 0; q < S / 2; ++q) w[q] = q1[q];
    }
  }
  __device__ __forceinline__ float operator[](int s) const {
    return (s & 1) ? __uint_as_float(w[s >> 1] & 0xffff0000u) : __uint_as_float(w[s >> 1] << 16);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < S / 2; ++q) w[q] = 0u;
  }
  // Force the words into SGPRs (after a load the compiler made per lane).
  __device__ __forceinline__ void uniform() {
#pragma unroll
    for (int q = 0; q < S / 2; ++q) w[q] = __builtin_amdgcn_readfirstlane(w[q]);
  }
};
template <int S> struct Row<float, S> {
  float w[S];
  __device__ __forceinline__ void load(const float* __restrict__ p) { load_row(w, p); }
  __device__ __forceinline__ float operator[](int s) const { return w[s]; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < S; ++q) w[q] = 0.0f;
  }
  __device__ __forceinline__ void uniform() {
#pragma unroll
    for (int q = 0; q < S; ++q) w[q] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w[q])));
  }
};

// DPP move within rows of 16 lanes (ctrl: quad_perm, row_ror, row_half_mirror ...).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Two adjacent B or C values of one token, read per lane (bf16 pairs packed in
// one dword), for the per-token products C_t . B_t.
template <class T> struct Pair;
template <> struct Pair<uint16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
  }
  __device__ __forceinline__ float dot(const Pair& o) const {
    return fmaf(__uint_as_float(w & 0xffff0000u), __uint_as_float(o.w & 0xffff0000u),
                __uint_as_float(w << 16) * __uint_as_float(o.w << 16));
  }
};
template <> struct Pair<float> {
  float a, b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
    b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4, 0, 0));
  }
  __device__ __forceinline__ float dot(const Pair& o) const { return fmaf(b, o.b, a * o.a); }
};

// Exponential-trapezoidal recurrence,
//   h_t = a_t h_{t-1} + dt_t ((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t),
// scanned as an Euler-form recurrence on the shifted state
//   g_t = h_t + w_{t+1} B_t,   w_{t+1} = dt_{t+1} (1 - lam_{t+1}) x_t,
// which satisfies g_t = a_t g_{t-1} + (dt_t lam_t x_t + w_{t+1}) B_t: the
// same per-state work as the Euler scan.  The output uses
// C_t . h_t = C_t . g_t - w_{t+1} (C_t . B_t), and after the last token of a
// sequence w = 0, so g = h there.  Before the first token,
// g_{-1} = h_{-1} + w_0 B_prev; trap_seed adds w_0 B_prev.
template <class T, int S, bool CONV, bool SP>
__device__ __forceinline__ void trap_seed(float (&h)[S], const ProArgs& pa, const Prologue<CONV, SP>& pro,
                                          const T* delta, int64_t b, int64_t L, int64_t d_inner, int64_t d,
                                          int n0) {
  const T* xp = static_cast<const T*>(pa.x_prev);
  const T* bp = static_cast<const T*>(pa.B_prev);
  if (!xp || !bp) return;
  const int64_t i0 = (b * L) * d_inner + d;                 // token 0 of sequence b
  const float dt0 = pro.dt(widen(delta[i0]));
  const float lam0 = pa.lam ? widen(static_cast<const T*>(pa.lam)[i0]) : 0.5f;
  const float w0 = dt0 * (1.0f - lam0) * widen(xp[b * d_inner + d]);
#pragma unroll
  for (int s = 0; s < S; ++s) h[s] = fmaf(w0, widen(bp[b * NSTATE + n0 + s]), h[s]);
}

// Addressing: a wave covers 64 consecutive channels [gbase, gbase + 64).  Row
// pointers (token t, channel gbase) are wave-uniform and live in SGPRs; a lane
// adds its own 32-bit offset `lo`.  Lanes past d_inner are clamped onto
// channel d_inner - 1 (they read valid memory and their results are dropped or
// duplicate that channel's).

// Streaming loads and stores are buffer instructions: a wave-uniform resource
// (SGPRs, based at the first row of the current token block), the lane's
// constant byte offset (VGPR) and the token's row offset (SGPR), so they cost
// no VALU address arithmetic.  A resource with num_records = 0 makes every
// load return 0 (out-of-range rule); it stands in for padding tokens' delta.
constexpr int kBufDword3 = 0x00020000;      // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int records = -1) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, records, kBufDword3);
}
__device__ __forceinline__ void buf_load(uint16_t& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  v = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_load(float& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t to_io(float v, uint16_t) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float to_io(float v, float) { return v; }

}  // namespace jscan_detail
