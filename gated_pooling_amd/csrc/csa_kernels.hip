// csa_kernels.hip -- gfx950 kernels of the CSA/HCA Compressor (THD-packed
// gated-softmax pooling), forward and backward.
//
// Sources (web pages): [PR5984] the NVIDIA/Megatron-LM pull request 5984
// page (squashed cudnn-frontend #427 commit log); [PR710] the cudnn-frontend
// pull request 710 page.
//
// Design (MI355X-first; the pages' kernels were written for another GPU and
// only their semantics are kept):
//   * The path is HBM-bound: per consumed kv/score slot it reads 4 bytes and
//     does ~20 fp32 VALU operations, far from any contraction, so there is no
//     MFMA.  Every consumed slot is read exactly once.
//   * Work item = (output row n, chunk of C output columns, C in {1, 2, 4}).
//     A lane owns one chunk and walks output rows grid-stride; lanes of a
//     wave take consecutive chunks, so each wave load covers contiguous bytes
//     of one half-row (256 bytes at C = 2).
//   * At coff = 2 a block's window is the previous block's first-half columns
//     plus its own second-half columns ([PR5984: fused forward+backward
//     commit]).  The lane loads exactly those 2*ratio half-row chunks, so no
//     slot is loaded twice and no block-to-block hand-off is needed.
//   * The window lives in VGPRs (ratio <= 4 keeps it to 2*4*C bf16 per
//     tensor); APE for the lane's chunk is loaded once per lane.  Ratio 128
//     has its own kernels (their section below), which stage each window in
//     LDS.
//   * Global memory goes through raw buffer instructions with exact byte
//     ranges: an index mistake cannot fault, out-of-range loads read 0 and
//     out-of-range stores are dropped.
//   * Backward stores are disjoint and atomic-free: the lane that owns a
//     window writes dkv/dscore for all of its slots; never-consumed slots get
//     +0.0 from one owner each ([PR5984: zero-init folding commit]): the
//     segment's last block writes its own first-half columns (coff = 2) and
//     the segment's seqlen % ratio tail rows; extra "zero" workgroups write
//     the rows of segments shorter than ratio and the rows past cu[S].
//   * dAPE: per-lane fp32 accumulators, reduced in a fixed order inside the
//     workgroup (staged in LDS, summed over the workgroup's row groups in
//     order), one partial row per workgroup in the workspace, then a second
//     kernel sums the partial rows in a fixed order.  Deterministic.
//   * The cu_seqlens -> output-block offset scan runs in each workgroup's
//     prologue (LDS) for up to kMaxLdsSegments segments; larger packs use a
//     one-workgroup scan kernel writing the offsets to the workspace; small
//     packs whose host copy of cu_seqlens the caller passes get the table in
//     the kernel arguments (no dependent global load before the first data
//     load).
//   * Floating point follows one fixed fp32 evaluation order (see
//     include/csa.h); the library is compiled with -ffp-contract=off so only
//     the explicit fmas below are fused.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "csa_launch.h"
#include "csa_walk.h"

namespace csa {
namespace {

using rsrc_t = __amdgpu_buffer_rsrc_t;
// Word 3 of a gfx9 raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}

// ---------------------------------------------------------------------------
// C bf16 values of one row chunk, as C/2 packed dwords (C = 1: the value in
// the low half of one dword).
// ---------------------------------------------------------------------------
template <int C>
struct Pack {
  uint32_t w[(C + 1) / 2];
};

// Columns of a chunk processed together by the softmax (2, or 1 at C = 1).
template <int C>
constexpr int kColGroup = C >= 2 ? 2 : 1;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Cache policy bits of buffer instructions: kAuxStream marks data that is
// touched once (kv/score/dout reads) as non-temporal, kAuxStreamStore the
// same for out/dkv/dscore writes.  Build knobs CSA_STREAM_HINT and
// CSA_STORE_HINT (0 disables a hint).
#ifndef CSA_STREAM_HINT
#define CSA_STREAM_HINT 2
#endif
#ifndef CSA_STORE_HINT
#define CSA_STORE_HINT CSA_STREAM_HINT
#endif
constexpr int kAuxStream = CSA_STREAM_HINT;
constexpr int kAuxStreamStore = CSA_STORE_HINT;

template <int C, int AUX = kAuxStream>
__device__ __forceinline__ Pack<C> load_pack(rsrc_t r, uint32_t byte_off) {
  Pack<C> p;
  if constexpr (C == 8) {
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX);
    p.w[0] = v.x; p.w[1] = v.y; p.w[2] = v.z; p.w[3] = v.w;
  } else if constexpr (C == 4) {
    u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, AUX);
    p.w[0] = v.x; p.w[1] = v.y;
  } else if constexpr (C == 2) {
    p.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, AUX);
  } else {
    static_assert(C == 1, "C must be 1, 2, 4 or 8");
    p.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, AUX);
  }
  return p;
}

template <int C, int AUX = kAuxStreamStore>
__device__ __forceinline__ void store_pack(rsrc_t r, uint32_t byte_off, const Pack<C>& p) {
  if constexpr (C == 8) {
    u32x4 v = {p.w[0], p.w[1], p.w[2], p.w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, AUX);
  } else if constexpr (C == 4) {
    u32x2 v = {p.w[0], p.w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, AUX);
  } else if constexpr (C == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(p.w[0], r, byte_off, 0, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(p.w[0]), r, byte_off, 0, AUX);
  }
}

// C consecutive fp32 values (APE row chunk).
template <int C>
__device__ __forceinline__ void load_f32(rsrc_t r, uint32_t byte_off, float (&out)[C]) {
  if constexpr (C == 8) {
    u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off + 16, 0, 0);
    out[0] = __uint_as_float(a.x); out[1] = __uint_as_float(a.y);
    out[2] = __uint_as_float(a.z); out[3] = __uint_as_float(a.w);
    out[4] = __uint_as_float(b.x); out[5] = __uint_as_float(b.y);
    out[6] = __uint_as_float(b.z); out[7] = __uint_as_float(b.w);
  } else if constexpr (C == 4) {
    u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    out[0] = __uint_as_float(a.x); out[1] = __uint_as_float(a.y);
    out[2] = __uint_as_float(a.z); out[3] = __uint_as_float(a.w);
  } else if constexpr (C == 2) {
    u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
    out[0] = __uint_as_float(a.x); out[1] = __uint_as_float(a.y);
  } else {
    out[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
  }
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
template <int C>
__device__ __forceinline__ float elem(const Pack<C>& p, int k) {
  const uint32_t w = p.w[k >> 1];
  return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
}

// Two fp32 -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// One column group's results packed as bf16: two columns, or one column in
// the low half (C = 1).
template <int NG>
__device__ __forceinline__ uint32_t pack_group(const float (&o)[NG]) {
  if constexpr (NG == 2) return pack_bf16x2(o[0], o[1]);
  else return pack_bf16x2(o[0], 0.0f);
}
template <int NG, int K>
__device__ __forceinline__ uint32_t pack_group_at(const float (&a)[NG][K], int i) {
  if constexpr (NG == 2) return pack_bf16x2(a[0][i], a[1][i]);
  else return pack_bf16x2(a[0][i], 0.0f);
}

// ---------------------------------------------------------------------------
// EXP: the fixed fp32 exponential of the evaluation order.
//   y >= -104 (clamp; e^-104 is below half the smallest subnormal),
//   k = rint(y log2 e), r = y - k ln2 in two fma steps (Cody-Waite with
//   ln2 split as fp32(ln2) + fp32(ln2 - fp32(ln2))), e^r by its degree-7
//   Taylor polynomial (Horner, coefficients fp32(1/n!)), scaled by 2^k.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float csa_exp(float y) {
  constexpr float kLog2e = 1.44269504088896340736f;
  constexpr float kLn2Hi = 0.693147180559945309417f;
  constexpr float kLn2Lo = -1.904654299957768e-09f;  // ln 2 - fp32(ln 2)
  y = fmaxf(y, -104.0f);
  const float k = __builtin_rintf(y * kLog2e);
  float r = __builtin_fmaf(-k, kLn2Hi, y);
  r = __builtin_fmaf(-k, kLn2Lo, r);
  float q = 1.0f / 5040.0f;
  q = __builtin_fmaf(q, r, 1.0f / 720.0f);
  q = __builtin_fmaf(q, r, 1.0f / 120.0f);
  q = __builtin_fmaf(q, r, 1.0f / 24.0f);
  q = __builtin_fmaf(q, r, 1.0f / 6.0f);
  q = __builtin_fmaf(q, r, 0.5f);
  q = __builtin_fmaf(q, r, 1.0f);
  q = __builtin_fmaf(q, r, 1.0f);
  return __builtin_ldexpf(q, static_cast<int>(k));
}

// One window, one column: weights e[], reciprocal R and the fp32 output o.
template <int K>
__device__ __forceinline__ float softmax_pool(const float (&x)[K], const float (&v)[K], float (&e)[K],
                                              float& R) {
  float m = x[0];
#pragma unroll
  for (int k = 1; k < K; ++k) m = fmaxf(m, x[k]);
#pragma unroll
  for (int k = 0; k < K; ++k) e[k] = csa_exp(x[k] - m);
  float Z = e[0];
#pragma unroll
  for (int k = 1; k < K; ++k) Z = Z + e[k];
  R = 1.0f / Z;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(e[k], v[k], acc);
  return acc * R;
}

// NC columns of one window at once, same arithmetic as softmax_pool per
// column.  Written stage by stage across all NC*K entries (each Horner step
// for every entry before the next step) so a wave has NC*K independent
// chains to issue instead of one long dependent chain per entry.
template <int NC, int K>
__device__ __forceinline__ void softmax_pool_cols(const float (&x)[NC][K], const float (&v)[NC][K],
                                                  float (&e)[NC][K], float (&R)[NC], float (&o)[NC]) {
  constexpr float kLog2e = 1.44269504088896340736f;
  constexpr float kLn2Hi = 0.693147180559945309417f;
  constexpr float kLn2Lo = -1.904654299957768e-09f;  // ln 2 - fp32(ln 2)
  float m[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) m[c] = x[c][0];
#pragma unroll
  for (int k = 1; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) m[c] = fmaxf(m[c], x[c][k]);
  float y[NC][K], kf[NC][K], q[NC][K];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) y[c][k] = fmaxf(x[c][k] - m[c], -104.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) kf[c][k] = __builtin_rintf(y[c][k] * kLog2e);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) y[c][k] = __builtin_fmaf(-kf[c][k], kLn2Hi, y[c][k]);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) y[c][k] = __builtin_fmaf(-kf[c][k], kLn2Lo, y[c][k]);  // y now holds r
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(1.0f / 5040.0f, y[c][k], 1.0f / 720.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 1.0f / 120.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 1.0f / 24.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 1.0f / 6.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 0.5f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 1.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][k] = __builtin_fmaf(q[c][k], y[c][k], 1.0f);
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) e[c][k] = __builtin_ldexpf(q[c][k], static_cast<int>(kf[c][k]));
  float Z[NC], acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    Z[c] = e[c][0];
    acc[c] = __builtin_fmaf(e[c][0], v[c][0], 0.0f);
  }
#pragma unroll
  for (int k = 1; k < K; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      Z[c] = Z[c] + e[c][k];
      acc[c] = __builtin_fmaf(e[c][k], v[c][k], acc[c]);
    }
#pragma unroll
  for (int c = 0; c < NC; ++c) R[c] = 1.0f / Z[c];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = acc[c] * R[c];
}

// ---------------------------------------------------------------------------
// Segment table: cu_seqlens and the exclusive scan of floor(L_s / ratio)
// (output-block offsets), validated.  Small packs: built per workgroup in
// LDS.  Large packs: read from the workspace (built by seg_scan_kernel).
// ---------------------------------------------------------------------------
struct SegTable {
  const int32_t* cu;
  const int32_t* off;
};

// Exclusive block-wide scan of int64 values; returns the block total.
template <int NT>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t& excl, int64_t* s_wave) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[wv] = incl;
  __syncthreads();
  int64_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int64_t t = s_wave[w];
    before += (w < wv) ? t : 0;
    total += t;
  }
  excl = before + incl - v;
  __syncthreads();  // s_wave may be reused by the caller
  return total;
}

// Returns true (uniformly across the block) iff cu is a valid pack for
// (S, T_cap, N).  The table location is a template parameter so lookups
// compile to ds_read (LDS) or global_load (workspace), never to flat loads,
// which would make every lookup wait for all outstanding buffer loads.
//   kTableLds:    built here in LDS from the device cu_seqlens (validated);
//                 LDS layout: int64 scratch[NT/64], cu[S+1], off[S+1].
//   kTableArgs:   copied to the same LDS layout from the kernel arguments
//                 (validated on the host): no global load before the first
//                 data load.
//   kTableGlobal: built in the workspace by seg_scan_kernel.
template <int R, int NT, int TBL>
__device__ bool load_segment_table(const SegParams& sp, int32_t* lds, SegTable& t) {
  if constexpr (TBL == kTableGlobal) {
    t.cu = sp.cu;
    t.off = sp.g_off;
    return __builtin_nontemporal_load(sp.g_flag) == 1;
  } else if constexpr (TBL == kTableArgs) {
    int32_t* s_cu = lds + 2 * (NT / 64);
    int32_t* s_off = s_cu + (sp.S + 1);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int i = 0; i <= kArgSegments; ++i) {
        if (i <= sp.S) {
          s_cu[i] = sp.arg_cu[i];
          s_off[i] = sp.arg_off[i];
        }
      }
    }
    __syncthreads();
    t.cu = s_cu;
    t.off = s_off;
    return true;
  } else {
    const int S = sp.S;
    int64_t* s_wave = reinterpret_cast<int64_t*>(lds);
    int32_t* s_cu = lds + 2 * (NT / 64);
    int32_t* s_off = s_cu + (S + 1);
    const int tid = threadIdx.x;
    for (int i = tid; i <= S; i += NT) s_cu[i] = sp.cu[i];
    __syncthreads();
    const int per = (S + NT - 1) / NT;
    const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
    int64_t local = 0;
    int bad = 0;
    for (int s = s0; s < s1; ++s) {
      const int32_t L = s_cu[s + 1] - s_cu[s];
      bad |= (L < 0);
      local += (L > 0) ? (L / R) : 0;
    }
    int64_t run;
    const int64_t total = block_exclusive_scan<NT>(local, run, s_wave);
    for (int s = s0; s < s1; ++s) {
      s_off[s] = static_cast<int32_t>(run);
      const int32_t L = s_cu[s + 1] - s_cu[s];
      run += (L > 0) ? (L / R) : 0;
    }
    if (tid == 0) {
      s_off[S] = static_cast<int32_t>(total);
      bad |= (s_cu[0] != 0) | (static_cast<int64_t>(s_cu[S]) > sp.T_cap) | (total != sp.N);
    }
    t.cu = s_cu;
    t.off = s_off;
    return __syncthreads_or(bad) == 0;
  }
}

// Largest s in [0, S) with off[s] <= n (requires n < off[S]); skips empty
// segments because they share their offset with the next segment.
__device__ __forceinline__ int find_segment(const int32_t* off, int S, int32_t n) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// One window's inputs, fetched one window ahead of its use.
//
// Every load of a window is issued before any of them is waited on, and the
// next window's loads are issued before the current window is computed, so
// each wave keeps two windows of loads in flight.  Loads a window does not
// need (the previous half of a segment's first block, lanes past the last
// output row) use an offset at the end of the buffer: the hardware range
// check returns 0 and touches no memory.
// ---------------------------------------------------------------------------
template <int R, int CO, int C, bool BWD>
struct Window {
  Pack<C> so[R], vo[R];                    // own rows (second half at coff 2)
  Pack<C> sp[CO == 2 ? R : 1];             // previous block's rows, first half
  Pack<C> vp[CO == 2 ? R : 1];
  Pack<C> gd[BWD ? 1 : 0 + 1];             // dout chunk (backward)
  uint32_t own;                            // first row of the block
  uint32_t seg_end;                        // cu[s + 1]
  bool has_prev;                           // coff 2 and not the segment's first block
  bool last;                               // the segment's last block
};

struct WinCtx {
  const int32_t* cu;
  const int32_t* off;
  int S;
  uint32_t N, W, d, g;
  uint32_t oob_io, oob_do;                 // past-the-end offsets (masked loads)
  rsrc_t rkv, rsc, rdo;
  bool active;                             // the lane's chunk is inside the row
};

template <int R, int CO, int C, bool BWD>
__device__ __forceinline__ void fetch_window(Window<R, CO, C, BWD>& w, uint32_t n, const WinCtx& x) {
  const bool valid = n < x.N;
  uint32_t own = 0, b = 0, nb = 0, end = 0;
  if (valid) {
    const int s = find_segment(x.off, x.S, static_cast<int32_t>(n));
    b = n - x.off[s];
    nb = x.off[s + 1] - x.off[s];
    own = x.cu[s] + b * R;
    end = x.cu[s + 1];
  }
  w.own = own;
  w.seg_end = end;
  w.has_prev = (CO == 2) && valid && b > 0;
  w.last = valid && (b + 1 == nb);
  const uint32_t col_own = (CO - 1) * x.d + x.g * C;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t o = (valid && x.active) ? ((own + i) * x.W + col_own) * 2u : x.oob_io;
    w.so[i] = load_pack<C>(x.rsc, o);
    w.vo[i] = load_pack<C>(x.rkv, o);
  }
  if constexpr (CO == 2) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t o = (w.has_prev && x.active) ? ((own - R + i) * x.W + x.g * C) * 2u : x.oob_io;
      w.sp[i] = load_pack<C>(x.rsc, o);
      w.vp[i] = load_pack<C>(x.rkv, o);
    }
  }
  if constexpr (BWD) w.gd[0] = load_pack<C>(x.rdo, (valid && x.active) ? (n * x.d + x.g * C) * 2u : x.oob_do);
}

// ---------------------------------------------------------------------------
// Wave-uniform windows.  When a row has at least 64 chunks, the 64 lanes of a
// wave work on the same output row, so the row's segment, first token row
// and flags are computed once per wave on the scalar unit (table entries
// read at uniform indices), and each load address is the lane's column
// offset plus a uniform row offset.  Masked loads use a uniform offset at
// the end of the buffer (the host keeps end + row bytes below 2^32).
// ---------------------------------------------------------------------------
// The segment table of a pack of fewer than 64 segments, held in registers:
// lane i of `cu` / `off` holds cu_seqlens[i] / the output-block offset of
// segment i (i <= S).  The uniform kernels build it per wave from the device
// cu_seqlens with one load and a wave prefix sum (no LDS, no barrier) and
// read entries with v_readlane.
struct RegTable {
  int32_t cu, off;
  bool on;
};

// Builds the register table; returns true (uniformly across the wave) iff cu
// is a valid pack for (S, T_cap, N), with the checks of load_segment_table.
template <int R>
__device__ __forceinline__ bool reg_segment_table(const SegParams& sp, RegTable& rt) {
  const int S = sp.S, lane = static_cast<int>(threadIdx.x & 63);
  const int32_t c = lane <= S ? sp.cu[lane] : 0;
  const int32_t L = __shfl_down(c, 1, 64) - c;                  // lane < S: segment length
  const int32_t nb = (lane < S && L > 0) ? L / R : 0;
  int32_t incl = nb;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const bool bad_len = lane < S && L < 0;
  const int32_t total = __builtin_amdgcn_readlane(incl, S);
  const int32_t c0 = __builtin_amdgcn_readlane(c, 0), cS = __builtin_amdgcn_readlane(c, S);
  rt.cu = c;
  rt.off = incl - nb;  // exclusive prefix; lane S: the total
  rt.on = true;
  return __ballot(bad_len) == 0 && c0 == 0 && static_cast<int64_t>(cS) <= sp.T_cap && total == sp.N;
}

// Entry i of a table in global memory that no kernel writes while this one
// runs (cu_seqlens, or the offsets seg_scan_kernel wrote before), read at a
// wave-uniform index through the scalar cache (constant address space): the
// row loop's lookups then wait on the scalar counter instead of the vector
// memory counter, which would also wait for every prefetched window.
__device__ __forceinline__ uint32_t scalar_entry(const int32_t* t, int i) {
  using const_ptr = const __attribute__((address_space(4))) int32_t*;
  return static_cast<uint32_t>(((const_ptr)t)[i]);
}

template <int TBL>
struct UTable {
  const SegParams& sp;   // kTableArgs: entries straight from the kernel arguments
  const int32_t* cu;     // otherwise: the table in LDS or in the workspace
  const int32_t* off;
  RegTable rt{0, 0, false};  // kTableLds with fewer than 64 segments: in registers
  __device__ __forceinline__ uint32_t cu_at(int i) const {
    if constexpr (TBL == kTableArgs) return static_cast<uint32_t>(sp.arg_cu[i]);
    else if constexpr (TBL == kTableGlobal) return scalar_entry(cu, i);
    else if (rt.on) return static_cast<uint32_t>(__builtin_amdgcn_readlane(rt.cu, i));
    else return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(cu[i]));
  }
  __device__ __forceinline__ uint32_t off_at(int i) const {
    if constexpr (TBL == kTableArgs) return static_cast<uint32_t>(sp.arg_off[i]);
    else if constexpr (TBL == kTableGlobal) return scalar_entry(off, i);
    else if (rt.on) return static_cast<uint32_t>(__builtin_amdgcn_readlane(rt.off, i));
    else return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(off[i]));
  }
};

struct WinCtxU {
  int S;
  uint32_t N, row_bytes, dout_row_bytes;
  uint32_t oob_io, oob_do;
  uint32_t lane_own, lane_prev, lane_gd;  // per-lane byte offsets inside a row
  rsrc_t rkv, rsc, rdo;
  bool active;                            // the lane's chunk is inside the row
};

// Fills w for output row n (uniform).  s_hint: a segment index <= the row's
// segment (rows only increase along a lane's walk); updated in place.
template <int R, int CO, int C, bool BWD, int TBL>
__device__ __forceinline__ void fetch_window_u(Window<R, CO, C, BWD>& w, uint32_t n, int& s_hint,
                                               const UTable<TBL>& t, const WinCtxU& x) {
  const bool valid = n < x.N;
  uint32_t own = 0, end = 0, b = 0, nb = 0;
  if (valid) {
    int lo = s_hint, hi = x.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (t.off_at(mid) <= n) lo = mid; else hi = mid - 1;
    }
    s_hint = lo;
    const uint32_t o0 = t.off_at(lo);
    b = n - o0;
    nb = t.off_at(lo + 1) - o0;
    own = t.cu_at(lo) + b * R;
    end = t.cu_at(lo + 1);
  }
  w.own = own;
  w.seg_end = end;
  w.has_prev = (CO == 2) && valid && b > 0;
  w.last = valid && (b + 1 == nb);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    uint32_t o = x.lane_own + (valid ? (own + i) * x.row_bytes : x.oob_io);
    o = x.active ? o : x.oob_io;
    w.so[i] = load_pack<C>(x.rsc, o);
    w.vo[i] = load_pack<C>(x.rkv, o);
  }
  if constexpr (CO == 2) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      uint32_t o = x.lane_prev + (w.has_prev ? (own - R + i) * x.row_bytes : x.oob_io);
      o = x.active ? o : x.oob_io;
      w.sp[i] = load_pack<C>(x.rsc, o);
      w.vp[i] = load_pack<C>(x.rkv, o);
    }
  }
  if constexpr (BWD)
    w.gd[0] = load_pack<C>(x.rdo, x.active ? x.lane_gd + (valid ? n * x.dout_row_bytes : x.oob_do) : x.oob_do);
}

// PF windows in flight along a lane's walk n, n + ns, n + 2 ns, ... < N:
// window k of the ring is computed while the next PF - 1 are loading.  The
// ring is unrolled, so each window keeps its own registers (no copies).
template <int PF, typename Win, typename Fetch, typename Body>
__device__ __forceinline__ void window_ring(uint32_t n, uint32_t ns, uint32_t N, Fetch&& fetch, Body&& body) {
  Win w[PF];
#pragma unroll
  for (int k = 0; k < PF - 1; ++k) fetch(w[k], n + k * ns);
  for (;;) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      fetch(w[(k + PF - 1) % PF], n + (PF - 1) * ns);
      body(w[k], n);
      n += ns;
      if (n >= N) return;
    }
  }
}

// Forward of one window: the C output columns packed as bf16.
template <int R, int CO, int C, bool BWD>
__device__ __forceinline__ Pack<C> fwd_window(const Window<R, CO, C, BWD>& w, const float (&ape_r)[CO][R][C]) {
  constexpr int NG = kColGroup<C>;
  Pack<C> outp;
  if (CO == 2 && w.has_prev) {
    constexpr int K = 2 * R;
#pragma unroll
    for (int kp = 0; kp < C / NG; ++kp) {
      float x[NG][K], v[NG][K], e[NG][K], Rz[NG], o2[NG];
#pragma unroll
      for (int hh = 0; hh < NG; ++hh) {
        const int k = NG * kp + hh;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          x[hh][i] = elem<C>(w.sp[i], k) + ape_r[0][i][k];
          v[hh][i] = elem<C>(w.vp[i], k);
          x[hh][R + i] = elem<C>(w.so[i], k) + ape_r[CO - 1][i][k];
          v[hh][R + i] = elem<C>(w.vo[i], k);
        }
      }
      softmax_pool_cols<NG, K>(x, v, e, Rz, o2);
      outp.w[kp] = pack_group<NG>(o2);
    }
  } else {
#pragma unroll
    for (int kp = 0; kp < C / NG; ++kp) {
      float x[NG][R], v[NG][R], e[NG][R], Rz[NG], o2[NG];
#pragma unroll
      for (int hh = 0; hh < NG; ++hh) {
        const int k = NG * kp + hh;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          x[hh][i] = elem<C>(w.so[i], k) + ape_r[CO - 1][i][k];
          v[hh][i] = elem<C>(w.vo[i], k);
        }
      }
      softmax_pool_cols<NG, R>(x, v, e, Rz, o2);
      outp.w[kp] = pack_group<NG>(o2);
    }
  }
  return outp;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int R, int CO, int C, int NT, int TBL, bool UNI, int PF, bool PAD>
__global__ __launch_bounds__(NT) void fwd_kernel(FwdParams p) {
  extern __shared__ int32_t lds[];
  SegTable tab{nullptr, nullptr};
  RegTable rt{0, 0, false};
  // the uniform path reads a kernel-argument table directly (no LDS copy) and
  // keeps a device table of fewer than 64 segments in registers
  if constexpr (UNI && TBL == kTableLds) {
    if (p.seg.S < 64) {
      if (!reg_segment_table<R>(p.seg, rt)) return;
    } else if (!load_segment_table<R, NT, TBL>(p.seg, lds, tab)) {
      return;
    }
  } else if constexpr (!(UNI && TBL == kTableArgs)) {
    if (!load_segment_table<R, NT, TBL>(p.seg, lds, tab)) return;
  }

  const uint32_t d = p.head_dim, W = CO * d;
  const uint32_t lgG = p.log2_chunks, G = 1u << lgG;
  const uint32_t L = blockIdx.x * NT + threadIdx.x;
  const uint32_t g = L & (G - 1);
  const uint32_t nstride = (gridDim.x * NT) >> lgG;
  const uint32_t N = static_cast<uint32_t>(p.seg.N);
  uint32_t n = L >> lgG;
  if constexpr (UNI) n = __builtin_amdgcn_readfirstlane(n);  // G >= 64: one row per wave
  if (n >= N || nstride == 0) return;
  // PAD: a row has p.chunks chunks, rounded up to G lanes; the extra lanes
  // load nothing (past-the-end offsets read 0) and store nothing
  const bool active = !PAD || g < p.chunks;

  const rsrc_t rkv = make_rsrc(p.kv, p.io_bytes);
  const rsrc_t rsc = make_rsrc(p.score, p.io_bytes);
  const rsrc_t rape = make_rsrc(p.ape, R * W * 4u);
  const rsrc_t rout = make_rsrc(p.out, N * d * 2u);
  const uint32_t oob_out = N * d * 2u;

  // APE of this chunk: [half][position][column]
  float ape_r[CO][R][C];
#pragma unroll
  for (int h = 0; h < CO; ++h)
#pragma unroll
    for (int i = 0; i < R; ++i) load_f32<C>(rape, active ? (i * W + h * d + g * C) * 4u : R * W * 4u, ape_r[h][i]);

  if constexpr (UNI) {
    const UTable<TBL> t{p.seg, tab.cu, tab.off, rt};
    WinCtxU x;
    x.S = p.seg.S;
    x.N = N;
    x.row_bytes = W * 2u;
    x.dout_row_bytes = 0;
    x.oob_io = p.io_bytes;
    x.oob_do = 0;
    x.lane_own = ((CO - 1) * d + g * C) * 2u;
    x.lane_prev = g * C * 2u;
    x.lane_gd = 0;
    x.rkv = rkv;
    x.rsc = rsc;
    x.rdo = rkv;
    x.active = active;
    const uint32_t lane_out = g * C * 2u, out_row = d * 2u;
    int s_hint = 0;
    using Win = Window<R, CO, C, false>;
    window_ring<PF, Win>(
        n, nstride, N, [&](Win& w, uint32_t m) { fetch_window_u(w, m, s_hint, t, x); },
        [&](const Win& w, uint32_t m) {
          store_pack<C>(rout, active ? m * out_row + lane_out : oob_out, fwd_window(w, ape_r));
        });
  } else {
    WinCtx x;
    x.cu = tab.cu;
    x.off = tab.off;
    x.S = p.seg.S;
    x.N = N;
    x.W = W;
    x.d = d;
    x.g = g;
    x.oob_io = p.io_bytes;
    x.oob_do = 0;
    x.rkv = rkv;
    x.rsc = rsc;
    x.rdo = rkv;
    x.active = active;
    Window<R, CO, C, false> cur, nxt;
    fetch_window(cur, n, x);
    for (; n < N; n += nstride) {
      fetch_window(nxt, n + nstride, x);
      store_pack<C>(rout, active ? (n * d + g * C) * 2u : oob_out, fwd_window(cur, ape_r));
      cur = nxt;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward: gradients, zero ownership, dAPE partials
// ---------------------------------------------------------------------------

// Ownership counting (builds with CSA_DEBUG_OWNERSHIP only): every store to
// dkv or dscore adds 1 to a uint32 counter per element it writes, so a test
// can check that each slot is written exactly once.  Stores at or past
// `limit` (masked lanes' past-the-end offsets) write nothing and count
// nothing.
__device__ __forceinline__ void own_count(uint32_t* cnt, uint32_t byte_off, uint32_t bytes, uint32_t limit) {
#ifdef CSA_DEBUG_OWNERSHIP
  if (cnt != nullptr && byte_off < limit)
    for (uint32_t e = 0; e < bytes / 2; ++e) atomicAdd(cnt + byte_off / 2 + e, 1u);
#else
  (void)cnt;
  (void)byte_off;
  (void)bytes;
  (void)limit;
#endif
}

// Zero a byte range [begin, end) of a buffer with 16-byte stores when both
// ends are 16-byte aligned, 4-byte stores when both are 4-byte aligned,
// 2-byte stores otherwise (rows of an odd coff * head_dim).  The walk steps
// an element index (walk_elements), so a range that ends near 2^32 bytes
// cannot wrap back onto the start of the buffer.
__device__ __forceinline__ void zero_range(rsrc_t r, uint32_t begin, uint32_t end, uint32_t first,
                                           uint32_t step, uint32_t* cnt, uint32_t limit) {
  if (((begin | end) & 15u) == 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    walk_elements<16>(begin, end, first, step, [&](uint32_t o) {
      __builtin_amdgcn_raw_buffer_store_b128(z, r, o, 0, 0);
      own_count(cnt, o, 16, limit);
    });
  } else if (((begin | end) & 3u) == 0) {
    walk_elements<4>(begin, end, first, step, [&](uint32_t o) {
      __builtin_amdgcn_raw_buffer_store_b32(0u, r, o, 0, 0);
      own_count(cnt, o, 4, limit);
    });
  } else {
    walk_elements<2>(begin, end, first, step, [&](uint32_t o) {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), r, o, 0, 0);
      own_count(cnt, o, 2, limit);
    });
  }
}

// Workgroup zid of nz zero-fills its share of the rows no window reads.
template <int R, int CO, int NT, typename Params>
__device__ void zero_sweep(const Params& p, const SegTable& tab, uint32_t zid, uint32_t nz) {
  const uint32_t W = CO * p.head_dim, row_bytes = W * 2u;
  const rsrc_t rdkv = make_rsrc(p.dkv, p.io_bytes);
  const rsrc_t rdsc = make_rsrc(p.dscore, p.io_bytes);
  const int S = p.seg.S;
  // rows of segments with no output block (L_s < ratio): whole rows
  for (int s = zid; s < S; s += nz) {
    if (tab.off[s + 1] == tab.off[s] && tab.cu[s + 1] > tab.cu[s]) {
      const uint32_t b0 = tab.cu[s] * row_bytes, b1 = tab.cu[s + 1] * row_bytes;
      zero_range(rdkv, b0, b1, threadIdx.x, NT, p.own_dkv, p.io_bytes);
      zero_range(rdsc, b0, b1, threadIdx.x, NT, p.own_dsc, p.io_bytes);
    }
  }
  // static-capacity padding rows past cu[S]
  const uint32_t b0 = tab.cu[S] * row_bytes, b1 = static_cast<uint32_t>(p.seg.T_cap) * row_bytes;
  zero_range(rdkv, b0, b1, zid * NT + threadIdx.x, nz * NT, p.own_dkv, p.io_bytes);
  zero_range(rdsc, b0, b1, zid * NT + threadIdx.x, nz * NT, p.own_dsc, p.io_bytes);
}

// The zero-fill workgroups [main_wgs, grid) of a launch share the sweep.
template <int R, int CO, int NT, typename Params>
__device__ void zero_sweep(const Params& p, const SegTable& tab) {
  zero_sweep<R, CO, NT>(p, tab, blockIdx.x - p.main_wgs, gridDim.x - p.main_wgs);
}

template <int R, int CO, int C, int NT, int TBL, bool UNI, int PF, bool PAD>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  extern __shared__ int32_t lds[];
  SegTable tab{nullptr, nullptr};
  RegTable rt{0, 0, false};
  bool valid = true;
  // the uniform path reads a kernel-argument table directly (no LDS copy) and
  // keeps a device table of fewer than 64 segments in registers; the
  // zero-fill workgroups still walk the table from LDS
  if constexpr (UNI && TBL == kTableArgs) {
    if (blockIdx.x >= p.main_wgs) load_segment_table<R, NT, TBL>(p.seg, lds, tab);
  } else if constexpr (UNI && TBL == kTableLds) {
    if (blockIdx.x >= p.main_wgs || p.seg.S >= 64) valid = load_segment_table<R, NT, TBL>(p.seg, lds, tab);
    else valid = reg_segment_table<R>(p.seg, rt);
  } else {
    valid = load_segment_table<R, NT, TBL>(p.seg, lds, tab);
  }
  if (TBL != kTableGlobal && blockIdx.x == 0 && threadIdx.x == 0)
    __builtin_nontemporal_store(valid ? 1 : 0, p.ws_flag);
  if (!valid) return;
  if (blockIdx.x >= p.main_wgs) {
    zero_sweep<R, CO, NT>(p, tab);
    return;
  }

  // Lane mapping: the G chunks of a row are split into slices of CS chunks
  // (CS * C * 2 >= 128 bytes, so a wave still reads whole cache lines).  A
  // workgroup owns one slice and NT / CS window rows at a time, so its dAPE
  // partial covers only its slice's columns: the partial buffer is
  // (workgroups per slice) x ratio x W floats instead of workgroups x ratio x W.
  const uint32_t d = p.head_dim, W = CO * d;
  const uint32_t lgG = p.log2_chunks;
  const uint32_t lgCS = p.log2_slice, CS = 1u << lgCS;
  const uint32_t lgSl = lgG - lgCS;                        // log2(slices)
  const uint32_t slice = blockIdx.x & ((1u << lgSl) - 1);
  const uint32_t wg_in_slice = blockIdx.x >> lgSl;
  const uint32_t wgs_per_slice = p.main_wgs >> lgSl;
  const uint32_t g = (slice << lgCS) + (threadIdx.x & (CS - 1));
  const uint32_t rows_per_wg = NT >> lgCS;
  const uint32_t nstride = wgs_per_slice * rows_per_wg;
  const uint32_t N = static_cast<uint32_t>(p.seg.N);

  const rsrc_t rkv = make_rsrc(p.kv, p.io_bytes);
  const rsrc_t rsc = make_rsrc(p.score, p.io_bytes);
  const rsrc_t rdkv = make_rsrc(p.dkv, p.io_bytes);
  const rsrc_t rdsc = make_rsrc(p.dscore, p.io_bytes);
  const rsrc_t rape = make_rsrc(p.ape, R * W * 4u);
  const rsrc_t rdo = make_rsrc(p.dout, N * d * 2u);
  // PAD: a row has p.chunks chunks, rounded up to the lanes of G; the extra
  // lanes load nothing (past-the-end offsets read 0, so their dAPE terms are
  // 0) and store nothing
  const bool active = !PAD || g < p.chunks;
  auto msk = [&](uint32_t o) { return active ? o : p.io_bytes; };
  // a gradient store (tensor 0: dkv, 1: dscore) of the lane's chunk
  auto put = [&](int tensor, uint32_t off, const Pack<C>& v) {
    store_pack<C>(tensor ? rdsc : rdkv, off, v);
    own_count(tensor ? p.own_dsc : p.own_dkv, off, C * 2, p.io_bytes);
  };

  float ape_r[CO][R][C];
  float acc_r[CO][R][C];
#pragma unroll
  for (int h = 0; h < CO; ++h)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      load_f32<C>(rape, active ? (i * W + h * d + g * C) * 4u : R * W * 4u, ape_r[h][i]);
#pragma unroll
      for (int k = 0; k < C; ++k) acc_r[h][i][k] = 0.0f;
    }

  const uint32_t rowb = W * 2u;
  const uint32_t lane_prev = g * C * 2u;                 // first-half column chunk
  const uint32_t lane_own = ((CO - 1) * d + g * C) * 2u;  // own-half column chunk

  // One window: gradients for its slots, dAPE accumulation, and (segment's
  // last block) the zeros of the never-read slots next to it.
  constexpr int NG = kColGroup<C>;
  auto body = [&](const Window<R, CO, C, true>& cur) {
    const uint32_t own = cur.own;
    const Pack<C>& gp = cur.gd[0];
    if (CO == 2 && cur.has_prev) {
      constexpr int K = 2 * R;
      Pack<C> gkv[K], gsc[K];
#pragma unroll
      for (int kp = 0; kp < C / NG; ++kp) {
        float a2[NG][K], ds2[NG][K];
        float xs[NG][K], v[NG][K], e[NG][K], Rz[NG], o2[NG];
#pragma unroll
        for (int hh = 0; hh < NG; ++hh) {
          const int k = NG * kp + hh;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            xs[hh][i] = elem<C>(cur.sp[i], k) + ape_r[0][i][k];
            v[hh][i] = elem<C>(cur.vp[i], k);
            xs[hh][R + i] = elem<C>(cur.so[i], k) + ape_r[CO - 1][i][k];
            v[hh][R + i] = elem<C>(cur.vo[i], k);
          }
        }
        softmax_pool_cols<NG, K>(xs, v, e, Rz, o2);
#pragma unroll
        for (int hh = 0; hh < NG; ++hh) {
          const int k = NG * kp + hh;
          const float Gk = Rz[hh] * elem<C>(gp, k);
#pragma unroll
          for (int i = 0; i < K; ++i) {
            const float a = e[hh][i] * Gk;
            const float ds = a * (v[hh][i] - o2[hh]);
            a2[hh][i] = a;
            ds2[hh][i] = ds;
          }
#pragma unroll
          for (int i = 0; i < R; ++i) {
            acc_r[0][i][k] += ds2[hh][i];
            acc_r[CO - 1][i][k] += ds2[hh][R + i];
          }
        }
#pragma unroll
        for (int i = 0; i < K; ++i) {
          gkv[i].w[kp] = pack_group_at<NG>(a2, i);
          gsc[i].w[kp] = pack_group_at<NG>(ds2, i);
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        put(0, msk((own - R + i) * rowb + lane_prev), gkv[i]);
        put(1, msk((own - R + i) * rowb + lane_prev), gsc[i]);
        put(0, msk((own + i) * rowb + lane_own), gkv[R + i]);
        put(1, msk((own + i) * rowb + lane_own), gsc[R + i]);
      }
    } else {
      Pack<C> gkv[R], gsc[R];
#pragma unroll
      for (int kp = 0; kp < C / NG; ++kp) {
        float a2[NG][R], ds2[NG][R];
        float xs[NG][R], v[NG][R], e[NG][R], Rz[NG], o2[NG];
#pragma unroll
        for (int hh = 0; hh < NG; ++hh) {
          const int k = NG * kp + hh;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            xs[hh][i] = elem<C>(cur.so[i], k) + ape_r[CO - 1][i][k];
            v[hh][i] = elem<C>(cur.vo[i], k);
          }
        }
        softmax_pool_cols<NG, R>(xs, v, e, Rz, o2);
#pragma unroll
        for (int hh = 0; hh < NG; ++hh) {
          const int k = NG * kp + hh;
          const float Gk = Rz[hh] * elem<C>(gp, k);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float a = e[hh][i] * Gk;
            const float ds = a * (v[hh][i] - o2[hh]);
            a2[hh][i] = a;
            ds2[hh][i] = ds;
            acc_r[CO - 1][i][k] += ds;
          }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          gkv[i].w[kp] = pack_group_at<NG>(a2, i);
          gsc[i].w[kp] = pack_group_at<NG>(ds2, i);
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        put(0, msk((own + i) * rowb + lane_own), gkv[i]);
        put(1, msk((own + i) * rowb + lane_own), gsc[i]);
      }
    }
    if (cur.last) {
      // The segment's last block owns the never-read slots next to it.
      Pack<C> z;
#pragma unroll
      for (int q = 0; q < (C + 1) / 2; ++q) z.w[q] = 0u;
      if (CO == 2) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          put(0, msk((own + i) * rowb + lane_prev), z);
          put(1, msk((own + i) * rowb + lane_prev), z);
        }
      }
      for (uint32_t t = own + R; t < cur.seg_end; ++t) {
#pragma unroll
        for (int h = 0; h < CO; ++h) {
          put(0, msk(t * rowb + h * d * 2u + lane_prev), z);
          put(1, msk(t * rowb + h * d * 2u + lane_prev), z);
        }
      }
    }
  };

  uint32_t n = wg_in_slice * rows_per_wg + (threadIdx.x >> lgCS);
  if constexpr (UNI) {
    // CS >= 64: the lanes of a wave share one row
    n = __builtin_amdgcn_readfirstlane(n);
    const UTable<TBL> t{p.seg, tab.cu, tab.off, rt};
    WinCtxU x;
    x.S = p.seg.S;
    x.N = N;
    x.row_bytes = rowb;
    x.dout_row_bytes = d * 2u;
    x.oob_io = p.io_bytes;
    x.oob_do = N * d * 2u;
    x.lane_own = lane_own;
    x.lane_prev = lane_prev;
    x.lane_gd = g * C * 2u;
    x.rkv = rkv;
    x.rsc = rsc;
    x.rdo = rdo;
    x.active = active;
    int s_hint = 0;
    if (n < N && nstride != 0) {
      using Win = Window<R, CO, C, true>;
      window_ring<PF, Win>(
          n, nstride, N, [&](Win& w, uint32_t m) { fetch_window_u(w, m, s_hint, t, x); },
          [&](const Win& w, uint32_t) { body(w); });
    }
  } else {
    WinCtx x;
    x.cu = tab.cu;
    x.off = tab.off;
    x.S = p.seg.S;
    x.N = N;
    x.W = W;
    x.d = d;
    x.g = g;
    x.oob_io = p.io_bytes;
    x.oob_do = N * d * 2u;
    x.rkv = rkv;
    x.rsc = rsc;
    x.rdo = rdo;
    x.active = active;
    Window<R, CO, C, true> cur, nxt;
    fetch_window(cur, n, x);
    for (; n < N && nstride != 0; n += nstride) {
      fetch_window(nxt, n + nstride, x);
      body(cur);
      cur = nxt;
    }
  }

  // ---- dAPE: fixed-order reduction inside the workgroup ----
  // Every thread stages its CO*R*C sums in LDS at stage[rg][h][i][gl*C + k]
  // (rg: the thread's row group, gl: its chunk in the slice).  After one
  // barrier, value q of the slice is the sum over row groups rg = 0, 1, ...
  // in that order (one barrier and no read-modify-write rounds: the tail
  // runs when every workgroup finishes at once, so it is on the critical
  // path).
  const uint32_t CW = CS * C;
  const uint32_t RG = NT >> lgCS;   // row groups of the workgroup
  const uint32_t QW = CO * R * CW;  // values of one row group
  float* stage = reinterpret_cast<float*>(lds + p.lds_table_words);
  {
    const uint32_t rg = threadIdx.x >> lgCS, gl = threadIdx.x & (CS - 1);
#pragma unroll
    for (int h = 0; h < CO; ++h)
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int k = 0; k < C; ++k) stage[rg * QW + (h * R + i) * CW + gl * C + k] = acc_r[h][i][k];
  }
  __syncthreads();
  // 3) one partial row per workgroup of a slice, stored in column blocks of
  //    kPartBlock floats: value j = i*W + h*d + col of partial row `row` is at
  //    ((j / kPartBlock) * rows + row) * kPartBlock + j % kPartBlock, so the
  //    reduce reads each column block as one contiguous run
  const uint32_t cbase = slice * CW;
  const uint32_t prow = p.partial_rows;
  const uint32_t nblk = (R * W + kPartBlock - 1) / kPartBlock;
  const rsrc_t rpart = make_rsrc(p.partials, nblk * prow * kPartBlock * 4u);
  if (!PAD && (d & 3u) == 0 && (CW & 3u) == 0) {
    // four consecutive values per step (same order of additions): 16-byte
    // LDS reads and one 16-byte store, which stays inside one column block
    // because j is a multiple of 4.  A thread takes at most CO*R*C/4 steps
    // (QW = CO*R*C*CS and CS <= NT); the steps are unrolled rather than
    // looped, so the stores do not make the compiler wait for every
    // outstanding store of the window loop first (it flushes the memory
    // counter ahead of a loop that stores).
#pragma unroll
    for (int step = 0; step < (CO * R * C + 3) / 4; ++step) {
      const uint32_t idx = (threadIdx.x + step * NT) * 4u;
      if (idx >= QW) break;
      const uint32_t hi = idx / CW, c = idx - hi * CW;
      const uint32_t h = hi / R, i = hi - h * R;
      f32x4 t = *reinterpret_cast<const f32x4*>(stage + idx);
      for (uint32_t g2 = 1; g2 < RG; ++g2) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(stage + g2 * QW + idx);
        t.x = t.x + u.x;
        t.y = t.y + u.y;
        t.z = t.z + u.z;
        t.w = t.w + u.w;
      }
      const uint32_t j = i * W + h * d + cbase + c;
      const uint32_t o = ((j / kPartBlock) * prow + wg_in_slice) * kPartBlock + (j % kPartBlock);
      const u32x4 v = {__float_as_uint(t.x), __float_as_uint(t.y), __float_as_uint(t.z), __float_as_uint(t.w)};
      __builtin_amdgcn_raw_buffer_store_b128(v, rpart, o * 4u, 0, 0);
    }
    return;
  }
  for (uint32_t idx = threadIdx.x; idx < QW; idx += NT) {
    const uint32_t hi = idx / CW, c = idx - hi * CW;
    const uint32_t h = hi / R, i = hi - h * R;
    if (PAD && cbase + c >= d) continue;  // padding lanes' columns
    float t = stage[idx];
    for (uint32_t g2 = 1; g2 < RG; ++g2) t = t + stage[g2 * QW + idx];
    const uint32_t j = i * W + h * d + cbase + c;
    const uint32_t o = ((j / kPartBlock) * prow + wg_in_slice) * kPartBlock + (j % kPartBlock);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(t), rpart, o * 4u, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// dAPE reduce: dape[j] = sum over partial rows, in a fixed order.
// A workgroup owns one column block (kPartBlock consecutive columns, stored
// contiguously for all partial rows).  Thread t takes the 4-column group
// (t mod 8) and the rows r = t/8, t/8 + 32, ... in increasing order (every
// load of the thread issued before the first add, so the block is one round
// trip from memory); the 32 row-group sums of a column are then added in
// row-group order through LDS.  The order depends only on the problem, not
// on timing: deterministic.
// ---------------------------------------------------------------------------
constexpr int kReduceNT = 256;
constexpr int kReduceQuads = kPartBlock / 4;               // 8 float4 per row
constexpr int kReduceGroups = kReduceNT / kReduceQuads;    // 32 row groups
constexpr int kReduceBatch = 8;

__global__ __launch_bounds__(kReduceNT) void dape_reduce_kernel(ReduceParams p) {
  __shared__ f32x4 part[kReduceGroups][kReduceQuads];
  const uint32_t q = threadIdx.x % kReduceQuads, rg = threadIdx.x / kReduceQuads;
  const uint32_t cols = p.cols, rows = p.rows;
  const uint32_t nblk = (cols + kPartBlock - 1) / kPartBlock;
  // the validity flag is loaded alongside the partials and checked before
  // anything is stored (bad cu_seqlens: dape is left untouched)
  const int32_t flag = __builtin_nontemporal_load(p.ws_flag);
  const uint32_t bytes = nblk * rows * kPartBlock * 4u;
  const rsrc_t rpart = make_rsrc(p.partials, bytes);
  const uint32_t base_off = (blockIdx.x * rows * kPartBlock + q * 4) * 4u;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (uint32_t base = rg; base < rows; base += kReduceGroups * kReduceBatch) {
    u32x4 v[kReduceBatch];
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      const uint32_t r = base + u * kReduceGroups;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rpart, r < rows ? base_off + r * kPartBlock * 4u : bytes, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kReduceBatch; ++u) {
      if (base + u * kReduceGroups < rows) {
        s.x = s.x + __uint_as_float(v[u].x);
        s.y = s.y + __uint_as_float(v[u].y);
        s.z = s.z + __uint_as_float(v[u].z);
        s.w = s.w + __uint_as_float(v[u].w);
      }
    }
  }
  part[rg][q] = s;
  __syncthreads();
  if (threadIdx.x < kPartBlock) {
    const uint32_t qq = threadIdx.x / 4, k = threadIdx.x % 4;
    const uint32_t col = blockIdx.x * kPartBlock + threadIdx.x;
    float t = part[0][qq][k];
#pragma unroll 8
    for (int g = 1; g < kReduceGroups; ++g) t = t + part[g][qq][k];
    if (col < cols && flag == 1) p.dape[col] = t;
  }
}

// ---------------------------------------------------------------------------
// ratio = 128 [PR5984: ratio=128 commit]: a window holds 128 * coff rows per
// column, too many for one lane's registers, so both kernels stage windows in
// LDS: a workgroup owns a slice of kSlice128 = 64 columns (lane = column) and
// walks output rows.  Each lane's window entries are split over the waves
// (16 per wave and half window in the forward, 8 coff per wave in the
// backward), and per row:
//   1. x = score + ape for the wave's entries, the wave's max, exchanged
//      through LDS -> the window max m (backward) or the max of each half
//      window (forward);
//   2. e = EXP(x - m); the entries' Z (adds) and acc (fma chain from 0) are
//      summed in chains of consecutive entries, then the chain sums in window
//      order; the forward merges its two halves by rescaling with EXP of the
//      difference of their maxima;
//   forward 3. out = acc * (1/Z) as bf16;
//   backward 3. a = e R g, ds = a (v - o) as bf16, written over the staged
//      inputs in LDS and stored with 16-byte stores; dAPE sums stay in
//      registers (a wave always holds the same positions of its slice) and
//      leave as one partial row per workgroup.
// These orders are not the single chain of the ratio 2 and 4 kernels: the
// pages hold ratio 128 to the final bf16 rounding instead of to bit equality
// [PR5984: ratio=128 commit, numerics contract per ratio family], and
// include/csa.h states the bound.  head_dim is a multiple of kSlice128, so
// every slice is whole.
// ---------------------------------------------------------------------------

// Byte offset in kv/score of window row k's slice, or `oob` when the row is
// masked (the previous half of a segment's first block).
template <int CO>
__device__ __forceinline__ uint32_t row128_offset(int k, uint32_t own, bool has_prev, uint32_t row_bytes,
                                                  uint32_t half_bytes, uint32_t slice_bytes, uint32_t oob) {
  if constexpr (CO == 2) {
    if (k < kRatio128) return has_prev ? (own - kRatio128 + k) * row_bytes + slice_bytes : oob;
    return (own + k - kRatio128) * row_bytes + half_bytes + slice_bytes;
  } else {
    return (own + k) * row_bytes + slice_bytes;
  }
}

// Row of output row n (uniform): segment lookup on the scalar unit.  `valid`
// is false for rows past the pack (the ring's look-ahead copies).
struct Row128 {
  uint32_t own, seg_end;
  bool has_prev, last, valid;
};
template <int TBL>
__device__ __forceinline__ Row128 row128(uint32_t n, uint32_t N, int& s_hint, const UTable<TBL>& t, int S) {
  Row128 r{};
  if (n >= N) return r;
  int lo = s_hint, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.off_at(mid) <= n) lo = mid; else hi = mid - 1;
  }
  s_hint = lo;
  const uint32_t o0 = t.off_at(lo), b = n - o0, nb = t.off_at(lo + 1) - o0;
  r.own = t.cu_at(lo) + b * kRatio128;
  r.seg_end = t.cu_at(lo + 1);
  r.has_prev = b > 0;
  r.last = b + 1 == nb;
  r.valid = true;
  return r;
}

// Forward: two workgroups per CU at coff 2 (four at coff 1), 4 * coff waves
// each.  A window is computed in two halves of kRows / 2 rows (coff 2: the
// previous block's rows, then the block's own rows; coff 1: the first and the
// last 64 rows), each half with its own maximum, and the halves are merged by
// rescaling, as the pages' forward merges per-chunk partials that carry their
// own maxima [PR5984: ratio=128 commit].  Per half h: m_h = max x over the
// half, e = EXP(x - m_h), Z_h and A_h the sums of e and e v (each wave a chain
// over its 16 entries, the wave sums added in wave order); then
// M = max(m_0, m_1), Z = Z_0 EXP(m_0 - M) + Z_1 EXP(m_1 - M), A likewise, and
// out = A (1/Z).  Halves are loaded with 16-byte loads into one of two
// register slots two halves ahead and written to one of two LDS stages while
// the previous half computes, so each workgroup keeps a window of loads in
// flight and a window's first half computes while its second half is still
// arriving.
template <int CO>
struct F128 {
  static constexpr int kRows = CO * kRatio128;              // window rows
  static constexpr int kHalfRows = kRows / 2;               // rows of a half window
  static constexpr int kWaves = fwd128_threads(CO) / 64;
  static constexpr int kThreads = fwd128_threads(CO);
  static constexpr int kE = kHalfRows / kWaves;             // entries per lane and half
  static constexpr int kParts = kSlice128 * 2 / 16;         // 16-byte parts of a row slice
  static constexpr int kIters = 2 * kHalfRows * kParts / kThreads;  // a thread's loads per half
  static constexpr int kRowsPerIter = kThreads / kParts;
  static constexpr int kHalfBytes = 2 * kHalfRows * kSlice128 * 2;  // score rows, then kv rows
  static_assert(2 * kHalfRows * kParts % kThreads == 0 && kIters % 2 == 0, "whole iterations");
  static_assert(2 * kHalfBytes == fwd128_stage_bytes(CO), "two stages");
  static_assert(3 * kWaves * kSlice128 * 4 == fwd128_red_bytes(CO), "exchange area");
};

// A thread's share of one half window, in registers.
template <int CO>
struct Half128 {
  u32x4 v[F128<CO>::kIters];
};

// Row of the half read by iteration it of this thread: iterations
// [0, kIters / 2) are score rows, the rest kv rows, so the buffer resource of
// each load is known at compile time.
template <int CO>
__device__ __forceinline__ int half_row128(int it) {
  using F = F128<CO>;
  return static_cast<int>(threadIdx.x / F::kParts) + (it % (F::kIters / 2)) * F::kRowsPerIter;
}

// Issue the loads of half h of row's window (no wait).  Rows past the pack
// and masked rows load from past the buffer's range and read zeros; every
// call issues the same loads, so the compiler's waits count a fixed number of
// loads between two halves.
template <int CO>
__device__ __forceinline__ void issue_half128(Half128<CO>& hv, rsrc_t rsc, rsrc_t rkv, const Row128& row, int h,
                                              uint32_t row_bytes, uint32_t half_bytes, uint32_t slice_bytes,
                                              uint32_t oob) {
  using F = F128<CO>;
  const uint32_t part = threadIdx.x % F::kParts;
#pragma unroll
  for (int it = 0; it < F::kIters; ++it) {
    const uint32_t o = row.valid ? row128_offset<CO>(h * F::kHalfRows + half_row128<CO>(it), row.own,
                                                     CO == 2 && row.has_prev, row_bytes, half_bytes, slice_bytes, oob)
                                 : oob;
    hv.v[it] = __builtin_amdgcn_raw_buffer_load_b128(it < F::kIters / 2 ? rsc : rkv, o == oob ? oob : o + part * 16u,
                                                     0, kAuxStream);
  }
}

// Write a thread's share of a half into an LDS stage (waits for its loads).
template <int CO>
__device__ __forceinline__ void write_half128(uint16_t* st, const Half128<CO>& hv) {
  using F = F128<CO>;
  const int part = threadIdx.x % F::kParts;
#pragma unroll
  for (int it = 0; it < F::kIters; ++it) {
    const int rq = (it / (F::kIters / 2)) * F::kHalfRows + half_row128<CO>(it);
    *reinterpret_cast<u32x4*>(st + rq * kSlice128 + part * 8) = hv.v[it];
  }
}

// One half from stage st (present is uniform across the workgroup): the
// wave's x = score + APE and its max into red; after a barrier, `mid` (the
// next half's LDS write and the loads after it), the half's max m, e =
// EXP(x - m) and the wave's Z and acc chains into red; after a second barrier
// wave 0 adds the wave sums in wave order into Z and A.  red holds the wave
// maxima, wave Z and wave acc, [kWaves][64] each.
template <int CO, typename Mid>
__device__ __forceinline__ void half128(const uint16_t* st, const float (&ape)[F128<CO>::kE], bool present, int wave,
                                        int lane, float* red, Mid&& mid, float& m, float& Z, float& A) {
  using F = F128<CO>;
  constexpr int E = F::kE, NW = F::kWaves, NC = kSlice128;
  const uint16_t* ss = st + wave * E * NC + lane;
  const uint16_t* sv = st + (F::kHalfRows + wave * E) * NC + lane;
  float x[E];
  if (present) {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __uint_as_float(uint32_t(ss[e * NC]) << 16) + ape[e];
    float mw = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) mw = fmaxf(mw, x[e]);
    red[wave * NC + lane] = mw;
  }
  __syncthreads();
  mid();
  if (present) {
    m = red[lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, red[w * NC + lane]);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = csa_exp(x[e] - m);
    float zl = x[0], al = 0.0f;
#pragma unroll
    for (int e = 1; e < E; ++e) zl = zl + x[e];
#pragma unroll
    for (int e = 0; e < E; ++e) al = __builtin_fmaf(x[e], __uint_as_float(uint32_t(sv[e * NC]) << 16), al);
    red[(NW + wave) * NC + lane] = zl;
    red[(2 * NW + wave) * NC + lane] = al;
  }
  __syncthreads();
  if (present && wave == 0) {
    Z = red[NW * NC + lane];
    A = red[2 * NW * NC + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      Z = Z + red[(NW + w) * NC + lane];
      A = A + red[(2 * NW + w) * NC + lane];
    }
  }
}

template <int CO, int TBL>
__global__ __launch_bounds__(F128<CO>::kThreads) void fwd128_kernel(Fwd128Params p) {
  using F = F128<CO>;
  constexpr int NT = F::kThreads, E = F::kE, NC = kSlice128;
  extern __shared__ int32_t lds[];
  SegTable tab{nullptr, nullptr};
  if constexpr (TBL != kTableArgs) {
    if (!load_segment_table<kRatio128, NT, TBL>(p.seg, lds, tab)) return;
  }
  // LDS: [table][two half-window stages][exchange]
  uint16_t* stage0 = reinterpret_cast<uint16_t*>(lds + p.lds_table_words);
  uint16_t* stage1 = stage0 + F::kHalfBytes / 2;
  float* red = reinterpret_cast<float*>(stage0 + F::kHalfBytes);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t d = p.head_dim, W = CO * d, N = static_cast<uint32_t>(p.seg.N);
  const uint32_t nslices = p.nslices, slice = blockIdx.x % nslices, per_slice = gridDim.x / nslices;
  const uint32_t col = slice * NC + lane;
  const rsrc_t rkv = make_rsrc(p.kv, p.io_bytes);
  const rsrc_t rsc = make_rsrc(p.score, p.io_bytes);
  const rsrc_t rape = make_rsrc(p.ape, kRatio128 * W * 4u);
  const rsrc_t rout = make_rsrc(p.out, N * d * 2u);
  // APE of the wave's entries: window row k = h kHalfRows + kE wave + e is
  // block position k mod 128 of the window's column half k / 128
  float ape_r[2][E];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = h * F::kHalfRows + wave * E + e;
      ape_r[h][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rape, ((k % kRatio128) * W + (CO == 2 ? k / kRatio128 : 0u) * d + col) * 4u, 0, 0));
    }

  const UTable<TBL> t{p.seg, tab.cu, tab.off};
  int s_hint = 0;
  const uint32_t row_bytes = W * 2u, half_bytes = d * 2u, slice_bytes = slice * NC * 2u, oob = p.io_bytes;
  uint32_t n = __builtin_amdgcn_readfirstlane(blockIdx.x / nslices);
  if (n >= N) return;
  // Slot h0 holds first halves, h1 second halves; r0, r1, r2: this row and
  // the next two of the workgroup
  Row128 r0 = row128<TBL>(n, N, s_hint, t, p.seg.S);
  Row128 r1 = row128<TBL>(n + per_slice, N, s_hint, t, p.seg.S);
  Half128<CO> h0, h1;
  issue_half128<CO>(h0, rsc, rkv, r0, 0, row_bytes, half_bytes, slice_bytes, oob);
  issue_half128<CO>(h1, rsc, rkv, r0, 1, row_bytes, half_bytes, slice_bytes, oob);
  write_half128<CO>(stage0, h0);
  issue_half128<CO>(h0, rsc, rkv, r1, 0, row_bytes, half_bytes, slice_bytes, oob);
  __syncthreads();
  for (;;) {
    const Row128 r2 = row128<TBL>(n + 2 * per_slice, N, s_hint, t, p.seg.S);
    float m0 = 0.0f, Z0 = 0.0f, A0 = 0.0f, m1 = 0.0f, Z1 = 0.0f, A1 = 0.0f;
    // the first half (absent in a segment's first block at coff 2); meanwhile
    // this row's second half goes to stage 1 and the next row's is loaded
    const bool first = !(CO == 2 && !r0.has_prev);
    half128<CO>(stage0, ape_r[0], first, wave, lane, red, [&] {
      write_half128<CO>(stage1, h1);
      issue_half128<CO>(h1, rsc, rkv, r1, 1, row_bytes, half_bytes, slice_bytes, oob);
    }, m0, Z0, A0);
    // the second half; meanwhile the next row's first half goes to stage 0
    // and the first half of the row after it is loaded
    half128<CO>(stage1, ape_r[1], true, wave, lane, red, [&] {
      write_half128<CO>(stage0, h0);
      issue_half128<CO>(h0, rsc, rkv, r2, 0, row_bytes, half_bytes, slice_bytes, oob);
    }, m1, Z1, A1);
    if (wave == 0) {
      float Z = Z1, A = A1;
      if (first) {
        const float M = fmaxf(m0, m1);
        const float s0 = csa_exp(m0 - M), s1 = csa_exp(m1 - M);
        Z = Z0 * s0 + Z1 * s1;
        A = A0 * s0 + A1 * s1;
      }
      const float o = A * (1.0f / Z);
      const Pack<1> ob{{pack_bf16x2(o, 0.0f)}};
      store_pack<1>(rout, (n * d + col) * 2u, ob);
    }
    n += per_slice;
    if (n >= N) break;
    r0 = r1;
    r1 = r2;
  }
}

// ---------------------------------------------------------------------------
// Backward (an "item" below is one output row of the workgroup's column
// slice): one workgroup of 16 waves per CU, wave w holding entries
// [8 coff w, 8 coff (w+1)) of its lane's column; each wave sums its entries
// in entry order, then the 16 wave sums are added in wave order.  Each row's
// window (score and kv, 128 bytes per window row) and dout slice are copied
// from memory into LDS by the buffer unit itself (buffer_load ... lds: no
// registers, no LDS write instructions) into one of two buffers while the
// previous row computes from the other, so the gradient arithmetic and
// stores of one row overlap the loads of the next.  The staged window is laid
// out by wave (wave w's score rows, then its kv rows), which is also what
// wave w copies, so a wave copies, reads, overwrites and stores only its own
// rows and the store needs no barrier.
//
// Waits.  An LDS copy counts in the issuing wave's vector-memory counter like
// a load and completes in issue order with the wave's other vector memory
// operations, so "row i's copy has landed" is `s_waitcnt vmcnt(k)` with k the
// number of vector memory operations this wave issued after that copy,
// followed by a barrier for the other waves' copies.  k is fixed by the code:
// every row issues the same copies and stores (copies past the last row and
// stores of masked rows use offsets past the buffer's range: the copy writes
// zeros, the store writes nothing); the segment-tail zero stores come after
// and only make a wait longer; the first row, with fewer operations behind
// it, waits for all.  There is no __syncthreads() in the row loop: its fence
// would wait for the copy in flight.
template <int CO>
struct R128 {
  static constexpr int kRows = CO * kRatio128;               // window entries per column
  static constexpr int kWaves = kThreads128 / 64;            // 16
  static constexpr int kCols = kSlice128;                    // columns of a row slice (lane = column)
  static constexpr int kE = kRows / kWaves;                  // entries per lane = window rows per wave
  static constexpr int kRowBytes = kCols * 2;                // one staged row slice: 128 bytes
  static constexpr int kWaveBytes = 2 * kE * kRowBytes;      // a wave's score rows then kv rows
  static constexpr int kCopies = kWaveBytes / 1024;          // 16-byte-per-lane copies per wave
  static constexpr int kStageBytes = kWaves * kWaveBytes;
  static constexpr int kBufBytes = kStageBytes + kRowBytes;  // + the dout row slice
  static constexpr int kBufs = 2;
  static_assert(kE % (1024 / kRowBytes) == 0, "a copy is one tensor's rows");
};

using lds_void_t = __attribute__((address_space(3))) void;

// Buffer descriptor words (as make_rsrc builds them) for the copies below,
// which take the descriptor as four scalar registers.
__device__ __forceinline__ u32x4 rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a))),
               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xFFFFu)),
               bytes, static_cast<uint32_t>(kRsrcWord3)};
}

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#endif
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its vector memory operations (copies in flight).
__device__ __forceinline__ void lds_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// One 16-byte-per-lane copy from a buffer into LDS (buffer_load_dwordx4 ...
// lds, non-temporal): active lane l's 16 bytes land at lds + 16 l (lds is
// wave-uniform, passed in M0); an out-of-range lane writes zeros.  Written in
// asm so that the compiler does not track the copy: its own wait insertion
// would otherwise wait for every copy in flight before each LDS read it
// cannot tell apart from a copy's target.  The copy has no register result;
// its completion is awaited explicitly (wait_vmem) before a barrier.  Nothing
// else in these kernels uses M0.  (The host pass of this file compiles an
// empty body that never runs.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: see above
__device__ __forceinline__ void lds_copy16(const u32x4& rsrc, const void* lds, uint32_t byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(base), "v"(byte_off), "s"(rsrc)
               : "memory", "m0");
#else
  (void)rsrc;
  (void)lds;
  (void)byte_off;
#endif
}
#pragma clang diagnostic pop

// The compiler tracks only its own loads: waiting for all of them (and the
// first items' copies, already issued) before the item loop keeps its waits
// for the APE registers out of the loop, where they would also wait for
// copies.
__device__ __forceinline__ void prologue_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Global byte offset of this lane's part of copy j of its wave (or oob):
// byte 1024 j + 16 lane of the wave's staged block is row slice
// r = (1024 j + 16 lane) / kRowBytes (score rows first, then kv rows), bytes
// 16 (lane % (kRowBytes / 16)) of it.
template <int CO>
__device__ __forceinline__ uint32_t copy_offset128(int j, const Row128& row, uint32_t row_bytes, uint32_t half_bytes,
                                                   uint32_t slice_bytes, uint32_t oob) {
  using Rw = R128<CO>;
  constexpr uint32_t kLanesPerRow = Rw::kRowBytes / 16;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t r = (1024u * j + 16u * lane) / Rw::kRowBytes, lr = r % Rw::kE;
  const int k = static_cast<int>(wave * Rw::kE + lr);
  if (!row.valid) return oob;
  const uint32_t o = row128_offset<CO>(k, row.own, CO == 2 && row.has_prev, row_bytes, half_bytes, slice_bytes, oob);
  return o == oob ? oob : o + (lane % kLanesPerRow) * 16u;
}
// tensor of copy j of a wave: score (0) or kv (1)
template <int CO>
__device__ __forceinline__ constexpr uint32_t copy_tensor128(int j) {
  return (1024u * j / R128<CO>::kRowBytes) / R128<CO>::kE;
}

// Issue the LDS copies of one item's window into `buf` (no wait); each copy
// is all score or all kv rows of the wave's block.
template <int CO>
__device__ __forceinline__ void copy_window128(uint8_t* buf, const u32x4& wsc, const u32x4& wkv, const Row128& row,
                                               uint32_t row_bytes, uint32_t half_bytes, uint32_t slice_bytes,
                                               uint32_t oob) {
  using Rw = R128<CO>;
  uint8_t* wb = buf + (threadIdx.x >> 6) * Rw::kWaveBytes;
#pragma unroll
  for (int j = 0; j < Rw::kCopies; ++j)
    lds_copy16(copy_tensor128<CO>(j) == 0 ? wsc : wkv, wb + 1024 * j,
               copy_offset128<CO>(j, row, row_bytes, half_bytes, slice_bytes, oob));
}

// 16-byte stores of a wave's staged block back to where copy j read it
// (masked rows: past the range, written nowhere).
template <int CO>
__device__ __forceinline__ void store_block128(const uint8_t* wb, int j, const Row128& row, rsrc_t rdsc, rsrc_t rdkv,
                                               uint32_t row_bytes, uint32_t half_bytes, uint32_t slice_bytes,
                                               uint32_t oob, uint32_t* own_dsc, uint32_t* own_dkv) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t o = copy_offset128<CO>(j, row, row_bytes, half_bytes, slice_bytes, oob);
  const u32x4 v = *reinterpret_cast<const u32x4*>(wb + 1024 * j + 16 * lane);
  constexpr bool kScore = copy_tensor128<CO>(0) == 0;
  (void)kScore;
  if (copy_tensor128<CO>(j) == 0) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rdsc, o, 0, kAuxStreamStore);
    own_count(own_dsc, o, 16, oob);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(v, rdkv, o, 0, kAuxStreamStore);
    own_count(own_dkv, o, 16, oob);
  }
}

// Window max of the lane's column: the lane's max, then the wave maxima
// through red[0, 16*64) (waves without entries pass -inf).
template <int CO>
__device__ __forceinline__ float window_max128(const float (&x)[R128<CO>::kE], bool present, int wave, int lane,
                                               float* red) {
  constexpr int E = R128<CO>::kE, NC = kSlice128;
  float mw = -__builtin_inff();
  if (present) {
    mw = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) mw = fmaxf(mw, x[e]);
  }
  red[wave * NC + lane] = mw;
  lds_barrier();
  float m = red[lane];
#pragma unroll
  for (int w = 1; w < R128<CO>::kWaves; ++w) m = fmaxf(m, red[w * NC + lane]);
  return m;
}

// e = EXP(x - m) in place; the lane's Z and acc chains into red (Z at
// [16*64, 32*64), acc at [32*64, 48*64)); waves without entries write 0.
template <int CO>
__device__ __forceinline__ void wave_sums128(float (&x)[R128<CO>::kE], const uint16_t* sv, float m, bool present,
                                             int wave, int lane, float* red) {
  constexpr int E = R128<CO>::kE, NC = kSlice128, NW = R128<CO>::kWaves;
  float zl = 0.0f, al = 0.0f;
  if (present) {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = csa_exp(x[e] - m);
    zl = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) zl = zl + x[e];
#pragma unroll
    for (int e = 0; e < E; ++e) al = __builtin_fmaf(x[e], __uint_as_float(uint32_t(sv[64 * e]) << 16), al);
  }
  red[(NW + wave) * NC + lane] = zl;
  red[(2 * NW + wave) * NC + lane] = al;
}

// Z and acc of the window: wave sums added in wave order from the first wave
// with entries (after the barrier that follows wave_sums128).
template <int CO>
__device__ __forceinline__ void window_sums128(bool has_prev, int lane, const float* red, float& Z, float& acc) {
  constexpr int NW = R128<CO>::kWaves, NC = kSlice128;
  const int w0 = (CO == 2 && !has_prev) ? NW / 2 : 0, c = lane;
  Z = red[(NW + w0) * NC + c];
  acc = red[(2 * NW + w0) * NC + c];
  for (int w = w0 + 1; w < NW; ++w) {
    Z = Z + red[(NW + w) * NC + c];
    acc = acc + red[(2 * NW + w) * NC + c];
  }
}

// Wait for item i's copies: after them this wave issued the copies of the
// next kBufs - 2 items (CP operations each) and, once i >= kBufs - 1, the
// stores of the kBufs - 1 previous items (ST each); earlier items wait for
// the copies alone (longer than needed, never shorter).
template <int CO, int CP, int ST>
__device__ __forceinline__ void wait_item(uint32_t i) {
  constexpr int NB = R128<CO>::kBufs;
  if (i + 1 >= NB) wait_vmem<(NB - 2) * CP + (NB - 1) * ST>();
  else wait_vmem<(NB - 2) * CP>();
}

template <int CO, int TBL>
__global__ __launch_bounds__(kThreads128) void bwd128_kernel(Bwd128Params p) {
  using Rw = R128<CO>;
  constexpr int NT = kThreads128, E = Rw::kE, NB = Rw::kBufs, NC = kSlice128;
  __shared__ __attribute__((aligned(16))) uint8_t ring[NB * Rw::kBufBytes];
  extern __shared__ int32_t lds[];  // [table][exchange]
  SegTable tab{nullptr, nullptr};
  // every workgroup walks the LDS table in the zero sweep after its items
  const bool valid = load_segment_table<kRatio128, NT, TBL>(p.seg, lds, tab);
  if (TBL != kTableGlobal && blockIdx.x == 0 && threadIdx.x == 0) __builtin_nontemporal_store(valid ? 1 : 0, p.ws_flag);
  if (!valid) return;
  float* red = reinterpret_cast<float*>(lds + p.lds_table_words);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t d = p.head_dim, W = CO * d, N = static_cast<uint32_t>(p.seg.N);
  const uint32_t nslices = p.nslices, slice = blockIdx.x % nslices, stride = gridDim.x / nslices;
  const uint32_t wg_in_slice = blockIdx.x / nslices;
  const uint32_t col = slice * NC + lane;
  const rsrc_t rdkv = make_rsrc(p.dkv, p.io_bytes);
  const rsrc_t rdsc = make_rsrc(p.dscore, p.io_bytes);
  const rsrc_t rape = make_rsrc(p.ape, kRatio128 * W * 4u);
  const u32x4 wkv = rsrc_words(p.kv, p.io_bytes), wsc = rsrc_words(p.score, p.io_bytes);
  const uint32_t dout_bytes = N * d * 2u;
  const u32x4 wdo = rsrc_words(p.dout, dout_bytes);
  const uint32_t kw = wave * Rw::kE, half = CO == 2 ? kw / kRatio128 : 0;
  const bool prev_half = CO == 2 && half == 0;
  float ape_r[E], dape_r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t pos = (kw + e) % kRatio128;
    ape_r[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rape, (pos * W + half * d + col) * 4u, 0, 0));
    dape_r[e] = 0.0f;
  }

  const UTable<TBL> t{p.seg, tab.cu, tab.off};
  int s_hint = 0;
  const uint32_t row_bytes = W * 2u, half_bytes = d * 2u, slice_bytes = slice * NC * 2u;
  // one item's copies: the window, and (wave 0, one 16-byte part per lane) the
  // dout row slice
  auto copy_item = [&](uint8_t* buf, const Row128& r, uint32_t nr) {
    copy_window128<CO>(buf, wsc, wkv, r, row_bytes, half_bytes, slice_bytes, p.io_bytes);
    if (wave == 0 && lane < Rw::kRowBytes / 16)
      lds_copy16(wdo, buf + Rw::kStageBytes, r.valid ? (nr * d + slice * NC) * 2u + lane * 16u : dout_bytes);
  };
  uint32_t n = __builtin_amdgcn_readfirstlane(wg_in_slice);
  if (n < N) {
    Row128 ahead[NB - 1];
#pragma unroll
    for (int a = 0; a < NB - 1; ++a) {
      ahead[a] = row128<TBL>(n + a * stride, N, s_hint, t, p.seg.S);
      copy_item(ring + a * Rw::kBufBytes, ahead[a], n + a * stride);
    }
    prologue_wait();
    for (uint32_t i = 0;; ++i) {
      uint8_t* cur = ring + (i % NB) * Rw::kBufBytes;
      // wave 0 issues one more copy per item (dout); every wave stores
      // kCopies gradient blocks per item
      if (wave == 0) wait_item<CO, Rw::kCopies + 1, Rw::kCopies>(i);
      else wait_item<CO, Rw::kCopies, Rw::kCopies>(i);
      lds_barrier();  // the item is in LDS; every wave is done with item i - 1
      const Row128 row = ahead[0];
      {
        const uint32_t nn = n + (NB - 1) * stride;
        const Row128 nxt = row128<TBL>(nn, N, s_hint, t, p.seg.S);
        copy_item(ring + ((i + NB - 1) % NB) * Rw::kBufBytes, nxt, nn);
#pragma unroll
        for (int a = 0; a < NB - 2; ++a) ahead[a] = ahead[a + 1];
        ahead[NB - 2] = nxt;
      }
      const bool present = !(prev_half && !row.has_prev);
      uint8_t* wb = cur + wave * Rw::kWaveBytes;
      uint16_t* sx = reinterpret_cast<uint16_t*>(wb) + lane;
      uint16_t* sv = sx + Rw::kE * NC;
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = __uint_as_float(uint32_t(sx[64 * e]) << 16) + ape_r[e];
      const float m = window_max128<CO>(x, present, wave, lane, red);
      wave_sums128<CO>(x, sv, m, present, wave, lane, red);
      lds_barrier();
      float Z, acc;
      window_sums128<CO>(row.has_prev, lane, red, Z, acc);
      const float g = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(cur + Rw::kStageBytes)[lane])
                                      << 16);
      const float R = 1.0f / Z;
      const float o = acc * R;
      const float G = R * g;
      if (present) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float v = __uint_as_float(uint32_t(sv[64 * e]) << 16);
          const float a = x[e] * G;
          const float ds = a * (v - o);
          dape_r[e] += ds;
          const uint32_t ab = pack_bf16x2(a, ds);
          sv[64 * e] = static_cast<uint16_t>(ab & 0xFFFFu);  // dKV over kv
          sx[64 * e] = static_cast<uint16_t>(ab >> 16);      // dScore over score
        }
      }
      // the wave's own staged rows go back where they came from (same wave:
      // its LDS writes above are ordered before these reads)
#pragma unroll
      for (int j = 0; j < Rw::kCopies; ++j)
        store_block128<CO>(wb, j, row, rdsc, rdkv, row_bytes, half_bytes, slice_bytes, p.io_bytes, p.own_dsc,
                           p.own_dkv);
      if (row.last) {
        // the segment's last block owns the never-read slots next to it: its
        // own rows' first half (coff 2) and the seqlen % 128 tail rows
        const u32x4 z = {0u, 0u, 0u, 0u};
        constexpr uint32_t kParts = NC * 2 / 16;
        const uint32_t tail = row.seg_end - (row.own + kRatio128);
        const uint32_t nz = (CO == 2 ? kRatio128 : 0) + tail * CO;  // row slices to zero
        for (uint32_t q = threadIdx.x; q < 2 * nz * kParts; q += NT) {
          const uint32_t part = q % kParts, rq = q / kParts;
          const uint32_t tensor = rq / nz, k = rq % nz;
          uint32_t o2;
          if (CO == 2 && k < kRatio128) {
            o2 = (row.own + k) * row_bytes + slice_bytes;
          } else {
            const uint32_t kt = k - (CO == 2 ? kRatio128 : 0);
            o2 = (row.own + kRatio128 + kt / CO) * row_bytes + (kt % CO) * half_bytes + slice_bytes;
          }
          __builtin_amdgcn_raw_buffer_store_b128(z, tensor ? rdkv : rdsc, o2 + part * 16u, 0, kAuxStreamStore);
          own_count(tensor ? p.own_dkv : p.own_dsc, o2 + part * 16u, 16, p.io_bytes);
        }
      }
      n += stride;
      if (n >= N) break;
    }
    wait_vmem<0>();  // the look-ahead copies land before the workgroup's LDS is released
  }
  // never-read rows outside every window (segments shorter than 128, rows
  // past cu[S]): shared by all workgroups
  zero_sweep<kRatio128, CO, NT>(p, tab, blockIdx.x, gridDim.x);
  // dAPE: one partial row per workgroup of a slice (column-block layout)
  const uint32_t prow = p.partial_rows;
  const uint32_t nblk = (kRatio128 * W + kPartBlock - 1) / kPartBlock;
  const rsrc_t rpart = make_rsrc(p.partials, nblk * prow * kPartBlock * 4u);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t pos = (kw + e) % kRatio128;
    const uint32_t j = pos * W + half * d + col;
    const uint32_t o2 = ((j / kPartBlock) * prow + wg_in_slice) * kPartBlock + (j % kPartBlock);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dape_r[e]), rpart, o2 * 4u, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Offset scan for packs with more than kMaxLdsSegments segments: one
// workgroup walks cu in chunks, writes off[0..S] and a validity flag.
// ---------------------------------------------------------------------------
constexpr int kScanNT = 1024;

template <int R>
__global__ __launch_bounds__(kScanNT) void seg_scan_kernel(SegParams sp, int32_t* off, int32_t* flag) {
  __shared__ int64_t s_wave[kScanNT / 64];
  __shared__ int s_bad;
  const int S = sp.S, tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int64_t carry = 0;
  for (int base = 0; base < S; base += kScanNT) {
    const int s = base + tid;
    int64_t nb = 0;
    if (s < S) {
      const int32_t L = sp.cu[s + 1] - sp.cu[s];
      if (L < 0) s_bad = 1;
      nb = (L > 0) ? (L / R) : 0;
    }
    int64_t excl;
    const int64_t total = block_exclusive_scan<kScanNT>(nb, excl, s_wave);
    if (s < S) off[s] = static_cast<int32_t>(carry + excl);
    carry += total;
  }
  __syncthreads();
  if (tid == 0) {
    off[S] = static_cast<int32_t>(carry);
    const bool bad = s_bad || sp.cu[0] != 0 || static_cast<int64_t>(sp.cu[S]) > sp.T_cap || carry != sp.N;
    *flag = bad ? 0 : 1;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int R, int CO, int C, bool UNI, int PF, bool PAD>
static void launch_fwd_rccu(const FwdParams& p, const LaunchShape& sh, hipStream_t st) {
  const dim3 grid(sh.grid), block(kFwdThreads);
  if (p.seg.table == kTableGlobal)
    hipLaunchKernelGGL((fwd_kernel<R, CO, C, kFwdThreads, kTableGlobal, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
  else if (p.seg.table == kTableArgs)
    hipLaunchKernelGGL((fwd_kernel<R, CO, C, kFwdThreads, kTableArgs, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
  else
    hipLaunchKernelGGL((fwd_kernel<R, CO, C, kFwdThreads, kTableLds, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
}

template <int R, int CO, int C>
static bool launch_fwd_rcc(const FwdParams& p, const LaunchShape& sh, hipStream_t st) {
  if (sh.pad) {
    // padded rows (head_dim / cols not a power of two, or one column per
    // lane): 1 or 2 columns, two windows in flight
    if constexpr (C <= 2) {
      if (sh.prefetch != 2) return false;
      if (sh.uniform)
        launch_fwd_rccu<R, CO, C, true, 2, true>(p, sh, st);
      else
        launch_fwd_rccu<R, CO, C, false, 2, true>(p, sh, st);
      return true;
    }
    return false;
  }
  if constexpr (C == 1) {
    return false;
  } else {
    if (!sh.uniform) {
      launch_fwd_rccu<R, CO, C, false, 2, false>(p, sh, st);
      return true;
    }
    switch (sh.prefetch) {
      case 2: launch_fwd_rccu<R, CO, C, true, 2, false>(p, sh, st); return true;
      case 3: launch_fwd_rccu<R, CO, C, true, 3, false>(p, sh, st); return true;
      case 4: launch_fwd_rccu<R, CO, C, true, 4, false>(p, sh, st); return true;
    }
    return false;
  }
}

template <int R, int CO, int C, int NT, bool UNI, int PF, bool PAD>
static void launch_bwd_rccnu(const BwdParams& p, const LaunchShape& sh, hipStream_t st) {
  const dim3 grid(sh.grid), block(NT);
  if (p.seg.table == kTableGlobal)
    hipLaunchKernelGGL((bwd_kernel<R, CO, C, NT, kTableGlobal, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
  else if (p.seg.table == kTableArgs)
    hipLaunchKernelGGL((bwd_kernel<R, CO, C, NT, kTableArgs, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
  else
    hipLaunchKernelGGL((bwd_kernel<R, CO, C, NT, kTableLds, UNI, PF, PAD>), grid, block, sh.lds_bytes, st, p);
}

template <int R, int CO, int C, int NT>
static bool launch_bwd_rccn(const BwdParams& p, const LaunchShape& sh, hipStream_t st) {
  if (sh.pad) {
    // padded rows: 1 or 2 columns, 256 threads, two windows in flight
    if constexpr (C <= 2 && NT == 256) {
      if (sh.prefetch != 2) return false;
      if (sh.uniform)
        launch_bwd_rccnu<R, CO, C, NT, true, 2, true>(p, sh, st);
      else
        launch_bwd_rccnu<R, CO, C, NT, false, 2, true>(p, sh, st);
      return true;
    }
    return false;
  }
  if constexpr (C == 1) {
    return false;
  } else {
    if (!sh.uniform) {
      launch_bwd_rccnu<R, CO, C, NT, false, 2, false>(p, sh, st);
      return true;
    }
    if constexpr (NT <= 512) {
      switch (sh.prefetch) {
        case 2: launch_bwd_rccnu<R, CO, C, NT, true, 2, false>(p, sh, st); return true;
        case 3: launch_bwd_rccnu<R, CO, C, NT, true, 3, false>(p, sh, st); return true;
        case 4: launch_bwd_rccnu<R, CO, C, NT, true, 4, false>(p, sh, st); return true;
      }
      return false;
    } else {
      // 1024-thread workgroups: deeper rings would not fit the registers
      if (sh.prefetch != 2) return false;
      launch_bwd_rccnu<R, CO, C, NT, true, 2, false>(p, sh, st);
      return true;
    }
  }
}

template <int R, int CO, int C>
static bool launch_bwd_rcc(const BwdParams& p, const LaunchShape& sh, hipStream_t st) {
  switch (sh.threads) {
    case 256: return launch_bwd_rccn<R, CO, C, 256>(p, sh, st);
    case 512: return launch_bwd_rccn<R, CO, C, 512>(p, sh, st);
    case 1024:
      // 4 columns per lane at 1024 threads would spill (the planner caps it)
      if constexpr (C != 4) return launch_bwd_rccn<R, CO, C, 1024>(p, sh, st);
      break;
  }
  return false;
}

template <int R, int CO>
static bool launch_fwd_rc(const FwdParams& p, const LaunchShape& sh, hipStream_t st) {
  switch (sh.cols) {
    case 4: return launch_fwd_rcc<R, CO, 4>(p, sh, st);
    case 2: return launch_fwd_rcc<R, CO, 2>(p, sh, st);
    case 1: return launch_fwd_rcc<R, CO, 1>(p, sh, st);
  }
  return false;
}

template <int R, int CO>
static bool launch_bwd_rc(const BwdParams& p, const LaunchShape& sh, hipStream_t st) {
  switch (sh.cols) {
    case 4: return launch_bwd_rcc<R, CO, 4>(p, sh, st);
    case 2: return launch_bwd_rcc<R, CO, 2>(p, sh, st);
    case 1: return launch_bwd_rcc<R, CO, 1>(p, sh, st);
  }
  return false;
}

bool launch_fwd(int ratio, int coff, const FwdParams& p, const LaunchShape& sh, hipStream_t st) {
  if (ratio == 4 && coff == 2) return launch_fwd_rc<4, 2>(p, sh, st);
  if (ratio == 4 && coff == 1) return launch_fwd_rc<4, 1>(p, sh, st);
  if (ratio == 2 && coff == 2) return launch_fwd_rc<2, 2>(p, sh, st);
  if (ratio == 2 && coff == 1) return launch_fwd_rc<2, 1>(p, sh, st);
  return false;
}

bool launch_bwd(int ratio, int coff, const BwdParams& p, const LaunchShape& sh, hipStream_t st) {
  if (ratio == 4 && coff == 2) return launch_bwd_rc<4, 2>(p, sh, st);
  if (ratio == 4 && coff == 1) return launch_bwd_rc<4, 1>(p, sh, st);
  if (ratio == 2 && coff == 2) return launch_bwd_rc<2, 2>(p, sh, st);
  if (ratio == 2 && coff == 1) return launch_bwd_rc<2, 1>(p, sh, st);
  return false;
}

template <int CO>
static void launch_fwd128_c(const Fwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st) {
  const dim3 g(grid), b(F128<CO>::kThreads);
  if (p.seg.table == kTableGlobal)
    hipLaunchKernelGGL((fwd128_kernel<CO, kTableGlobal>), g, b, lds_bytes, st, p);
  else if (p.seg.table == kTableArgs)
    hipLaunchKernelGGL((fwd128_kernel<CO, kTableArgs>), g, b, lds_bytes, st, p);
  else
    hipLaunchKernelGGL((fwd128_kernel<CO, kTableLds>), g, b, lds_bytes, st, p);
}

template <int CO>
static void launch_bwd128_c(const Bwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st) {
  const dim3 g(grid), b(kThreads128);
  if (p.seg.table == kTableGlobal)
    hipLaunchKernelGGL((bwd128_kernel<CO, kTableGlobal>), g, b, lds_bytes, st, p);
  else if (p.seg.table == kTableArgs)
    hipLaunchKernelGGL((bwd128_kernel<CO, kTableArgs>), g, b, lds_bytes, st, p);
  else
    hipLaunchKernelGGL((bwd128_kernel<CO, kTableLds>), g, b, lds_bytes, st, p);
}

bool launch_fwd128(int coff, const Fwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st) {
  if (coff == 2) launch_fwd128_c<2>(p, grid, lds_bytes, st);
  else if (coff == 1) launch_fwd128_c<1>(p, grid, lds_bytes, st);
  else return false;
  return true;
}

bool launch_bwd128(int coff, const Bwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st) {
  if (coff == 2) launch_bwd128_c<2>(p, grid, lds_bytes, st);
  else if (coff == 1) launch_bwd128_c<1>(p, grid, lds_bytes, st);
  else return false;
  return true;
}

void launch_dape_reduce(const ReduceParams& p, hipStream_t st) {
  const uint32_t grid = (p.cols + kPartBlock - 1) / kPartBlock;
  hipLaunchKernelGGL(dape_reduce_kernel, dim3(grid), dim3(kReduceNT), 0, st, p);
}

bool launch_seg_scan(int ratio, const SegParams& sp, int32_t* off, int32_t* flag, hipStream_t st) {
  if (ratio == 4) {
    hipLaunchKernelGGL(seg_scan_kernel<4>, dim3(1), dim3(kScanNT), 0, st, sp, off, flag);
    return true;
  }
  if (ratio == 2) {
    hipLaunchKernelGGL(seg_scan_kernel<2>, dim3(1), dim3(kScanNT), 0, st, sp, off, flag);
    return true;
  }
  if (ratio == kRatio128) {
    hipLaunchKernelGGL(seg_scan_kernel<kRatio128>, dim3(1), dim3(kScanNT), 0, st, sp, off, flag);
    return true;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Scratch owned by the library, for the backward entry point that allocates
// nothing (csa_compressor_bwd_noalloc): the workspace of the ordinary entry
// point (validity flag, segment table, dAPE partials) lives here instead.
// Each GPU the library runs on holds its own copy from the module's load
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels receive the address that hipGetSymbolAddress
// returns for the current device, looked up once per device and cached.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace csa
