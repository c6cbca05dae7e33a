// csa_api.cpp -- the C ABI of libcsa (include/csa.h): argument validation,
// launch planning and dispatch to the gfx950 kernels.
//
// Validation and planning are pure host code and depend only on the problem
// description and the tuning knobs below, never on the device, so every
// rejection (including an undersized workspace) happens before any HIP call.
//
// Support envelope ([PR5984] = NVIDIA/Megatron-LM pull request 5984 page,
// [PR710] = cudnn-frontend pull request 710 page): ratio in {2, 4}
// ([PR710: What]) and 128 with head_dim a multiple of 64 ([PR5984: ratio=128
// commit]), coff in {1, 2} ([PR5984: coff commit]); the size limits
// total_tokens*coff*head_dim, total_comp*head_dim and ratio*coff*head_dim
// below 2^31 each, and the rejection of total_comp > 0 with
// total_tokens < ratio ([PR5984: review-feedback commit; PR710: What]).
// head_dim may be any value in [1, 1024]: an odd head_dim takes one column
// per lane (16-bit accesses), and a row whose chunk count is not a power of
// two is padded to the next power of two in lanes (the extra lanes are
// masked) [PR5984: vectorize-forward commit (scalar instantiation for odd
// head_dims)].
//
// Tuning knobs (environment, read once per process; every value is
// validated and falls back to the default):
//   CSA_FWD_COLS      output columns per lane in the forward (2, 4)
//   CSA_FWD_MAX_WGS   forward grid cap in workgroups of 256 threads
//                     (default 768 at ratio 4, 1024 at ratio 2)
//   CSA_BWD_COLS      output columns per lane in the backward (2, 4)
//   CSA_BWD_THREADS   backward workgroup size (256, 512, 1024)
//   CSA_BWD_MAX_WGS   backward grid cap in main workgroups (default 256 at
//                     ratio 4, 512 at ratio 2)
//   CSA_BWD_SLICE_BYTES  bytes of a half-row one backward workgroup covers
//                     (>= 128; smaller slices shrink the dAPE partials); the
//                     chunk count it gives is rounded down to a power of two,
//                     the only slice shape the kernels' lane mapping supports
//   CSA_UNIFORM       1: wave-uniform row path where a row has >= 64 chunks
//   CSA_FWD_PREFETCH, CSA_BWD_PREFETCH  windows in flight per lane on the
//                     uniform path (2, 3, 4)
//   CSA_R128_FWD_WGS, CSA_R128_BWD_WGS  ratio-128 grid caps (default: the
//                     workgroups the chip holds at once)

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "../../include/csa.h"
#include "csa_launch.h"

namespace {

thread_local std::string g_err;

#ifdef CSA_DEBUG_OWNERSHIP
// Ownership counters of the debug build (csa_debug_ownership_counters).
uint32_t* g_own_dkv = nullptr;
uint32_t* g_own_dsc = nullptr;
#endif

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

csa_status_t ok() {
  g_err.clear();
  return CSA_STATUS_SUCCESS;
}

struct Tuning {
  int fwd_cols = 2;
  int fwd_max_wgs = 0;    // 0: by ratio (see make_plan)
  int bwd_cols = 2;
  int bwd_threads = 256;
  int bwd_max_wgs = 0;    // 0: by ratio (see make_plan)
  int bwd_slice_bytes = 512;
  int uniform = 1;        // wave-uniform row path where a row has >= 64 chunks
  int fwd_prefetch = 2;   // windows in flight per lane (uniform path)
  int bwd_prefetch = 3;
  int r128_fwd_wgs = 0;   // ratio 128 grid caps (workgroups); 0: the chip's residency
  int r128_bwd_wgs = 0;
};

int env_int(const char* name, int dflt, const int* allowed, int n_allowed, int lo, int hi) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  long x = strtol(v, &end, 10);
  if (*end != '\0') return dflt;
  if (allowed) {
    for (int i = 0; i < n_allowed; ++i)
      if (allowed[i] == x) return static_cast<int>(x);
    return dflt;
  }
  return (x >= lo && x <= hi) ? static_cast<int>(x) : dflt;
}

const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning d;
    static const int cols[] = {2, 4};
    static const int threads[] = {256, 512, 1024};
    d.fwd_cols = env_int("CSA_FWD_COLS", d.fwd_cols, cols, 2, 0, 0);
    d.fwd_max_wgs = env_int("CSA_FWD_MAX_WGS", d.fwd_max_wgs, nullptr, 0, 1, 1 << 20);
    d.bwd_cols = env_int("CSA_BWD_COLS", d.bwd_cols, cols, 2, 0, 0);
    d.bwd_threads = env_int("CSA_BWD_THREADS", d.bwd_threads, threads, 3, 0, 0);
    d.bwd_max_wgs = env_int("CSA_BWD_MAX_WGS", d.bwd_max_wgs, nullptr, 0, 1, 1 << 16);
    d.bwd_slice_bytes = env_int("CSA_BWD_SLICE_BYTES", d.bwd_slice_bytes, nullptr, 0, 16, 1 << 16);
    d.uniform = env_int("CSA_UNIFORM", d.uniform, nullptr, 0, 0, 1);
    d.fwd_prefetch = env_int("CSA_FWD_PREFETCH", d.fwd_prefetch, nullptr, 0, 2, 4);
    d.bwd_prefetch = env_int("CSA_BWD_PREFETCH", d.bwd_prefetch, nullptr, 0, 2, 4);
    d.r128_fwd_wgs = env_int("CSA_R128_FWD_WGS", d.r128_fwd_wgs, nullptr, 0, 1, 1 << 20);
    d.r128_bwd_wgs = env_int("CSA_R128_BWD_WGS", d.r128_bwd_wgs, nullptr, 0, 1, 1 << 16);
    return d;
  }();
  return t;
}

struct Problem {
  int32_t ratio, coff, head_dim, S;
  int64_t T, N;
};

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int l = 0;
  while ((int64_t{1} << l) < x) ++l;
  return l;
}
uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

csa_status_t check_problem(const Problem& p) {
  if (p.ratio != 2 && p.ratio != 4 && p.ratio != csa::kRatio128)
    return fail(CSA_STATUS_NOT_SUPPORTED, "ratio must be 2, 4 or 128 (got %d)", p.ratio);
  if (p.coff != 1 && p.coff != 2)
    return fail(CSA_STATUS_NOT_SUPPORTED, "coff must be 1 or 2 (got %d)", p.coff);
  if (p.head_dim < 1 || p.head_dim > 1024)
    return fail(CSA_STATUS_NOT_SUPPORTED, "head_dim must be in [1, 1024] (got %d)", p.head_dim);
  if (p.ratio == csa::kRatio128 && p.head_dim % csa::kSlice128 != 0)
    return fail(CSA_STATUS_NOT_SUPPORTED, "ratio 128 needs head_dim a multiple of %d (got %d)", csa::kSlice128,
                p.head_dim);
  if (p.S < 0 || p.T < 0 || p.N < 0)
    return fail(CSA_STATUS_INVALID_VALUE, "negative size: num_segments=%d total_tokens=%lld total_comp=%lld",
                p.S, (long long)p.T, (long long)p.N);
  const int64_t W = int64_t{p.coff} * p.head_dim;
  const int64_t lim = int64_t{1} << 31;
  // (total_tokens + 1): a masked load's offset, one row past the end, must
  // still fit in 32 bits
  if ((p.T + 1) * W >= lim)
    return fail(CSA_STATUS_NOT_SUPPORTED, "(total_tokens+1)*coff*head_dim must be below 2^31");
  if (p.N * p.head_dim >= lim)
    return fail(CSA_STATUS_NOT_SUPPORTED, "total_comp*head_dim must be below 2^31");
  if (int64_t{p.ratio} * W >= lim)
    return fail(CSA_STATUS_NOT_SUPPORTED, "ratio*coff*head_dim must be below 2^31");
  if (p.N > 0 && p.T < p.ratio)
    return fail(CSA_STATUS_INVALID_VALUE, "total_comp > 0 with total_tokens < ratio");
  if (p.N * p.ratio > p.T)
    return fail(CSA_STATUS_INVALID_VALUE, "total_comp*ratio exceeds total_tokens");
  if (p.S == 0 && p.N != 0)
    return fail(CSA_STATUS_INVALID_VALUE, "total_comp > 0 with no segments");
  return ok();
}

// Workspace layout: [0, 256) header (int32 validity flag at 0);
// then, for packs above kMaxLdsSegments, int32 offsets [S + 1];
// then (backward) fp32 dAPE partials in column blocks
// [ceil(ratio*W / kPartBlock)][partial_rows][kPartBlock].
struct Plan {
  bool global_table;
  uint64_t off_bytes;   // offsets section size
  // forward
  csa::LaunchShape fwd;
  int fwd_log2_chunks;
  uint32_t fwd_chunks;
  uint64_t ws_fwd;
  // backward
  csa::LaunchShape bwd;
  int bwd_log2_chunks;
  uint32_t bwd_chunks;
  int bwd_log2_slice;
  uint32_t bwd_main_wgs;
  uint32_t partial_rows;
  uint32_t lds_table_words;
  uint64_t partial_offset;
  uint64_t ws_bwd;
  // ratio 128
  uint32_t nslices;
  uint32_t fwd_lds_table_words;
};

constexpr uint64_t kHeaderBytes = 256;

// Columns per lane: 1 for an odd head_dim; otherwise the requested 2 or 4
// when it divides head_dim into a power-of-two number of chunks, else 2.
int choose_cols(int head_dim, int want) {
  if (head_dim & 1) return 1;
  if (want == 4 && (head_dim % 4 != 0 || !is_pow2(head_dim / 4))) return 2;
  return want;
}
int64_t pow2_ceil(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
int64_t pow2_floor(int64_t x) {
  int64_t p = 1;
  while (2 * p <= x) p <<= 1;
  return p;
}

// ratio 128: a workgroup per (column slice, group of output rows), rows of a
// slice dealt round-robin to its workgroups (see the kernels).
//   forward: 4 * coff waves per workgroup, two half-window stages and the
//     exchange area in dynamic LDS after the segment table; two workgroups
//     per CU at coff 2, four at coff 1 (measured best on 65536-token packs);
//   backward: 1024 threads, one workgroup per CU (its two static LDS window
//     buffers take most of the CU's LDS); every workgroup also zero-fills a
//     share of the never-read rows after its windows, so there are no
//     separate zero-fill workgroups.  Dynamic LDS: the segment table and the
//     exchange area.
Plan make_plan_r128(const Problem& p) {
  const Tuning& tu = tuning();
  Plan pl{};
  const int64_t W = int64_t{p.coff} * p.head_dim;
  pl.global_table = p.S > csa::kMaxLdsSegments;
  pl.off_bytes = pl.global_table ? align_up(uint64_t(p.S + 1) * 4, 256) : 0;
  // int64 scan scratch [NT/64], cu [S+1], off [S+1]; keeps what follows it
  // 16-byte aligned
  auto table_words = [&](int NT) {
    return pl.global_table ? 0u : static_cast<uint32_t>(align_up(2 * (NT / 64) + 2 * uint64_t(p.S + 1), 4));
  };
  pl.nslices = static_cast<uint32_t>(p.head_dim / csa::kSlice128);
  const int64_t out_rows = p.N > 0 ? p.N : 1;
  auto per_slice = [&](int cap) {
    int64_t per = cap / pl.nslices;
    if (per < 1) per = 1;
    if (per > out_rows) per = out_rows;
    return per;
  };
  {
    const int NT = csa::fwd128_threads(p.coff);
    const int64_t per = per_slice(tu.r128_fwd_wgs ? tu.r128_fwd_wgs : (p.coff == 2 ? 2 : 4) * csa::kCUs);
    pl.fwd.grid = static_cast<uint32_t>(per * pl.nslices);
    pl.fwd.threads = NT;
    pl.fwd.cols = 1;
    pl.fwd_lds_table_words = table_words(NT);
    pl.fwd.lds_bytes = pl.fwd_lds_table_words * 4ull + csa::fwd128_stage_bytes(p.coff) +
                       csa::fwd128_red_bytes(p.coff);
    pl.ws_fwd = pl.global_table ? kHeaderBytes + pl.off_bytes : 0;
  }
  {
    const int64_t per = per_slice(tu.r128_bwd_wgs ? tu.r128_bwd_wgs : csa::kCUs);
    const int64_t main = per * pl.nslices;
    pl.bwd.grid = static_cast<uint32_t>(main);
    pl.bwd.threads = csa::kThreads128;
    pl.bwd.cols = 1;
    pl.bwd_main_wgs = static_cast<uint32_t>(main);
    pl.partial_rows = static_cast<uint32_t>(per);
    pl.lds_table_words = table_words(csa::kThreads128);
    pl.bwd.lds_bytes = pl.lds_table_words * 4ull + csa::kRed128Bytes;
    pl.partial_offset = kHeaderBytes + pl.off_bytes;
    const uint64_t nblk = (uint64_t(p.ratio) * W + csa::kPartBlock - 1) / csa::kPartBlock;
    pl.ws_bwd = pl.partial_offset + align_up(nblk * pl.partial_rows * csa::kPartBlock * 4, 256);
  }
  return pl;
}

Plan make_plan(const Problem& p) {
  if (p.ratio == csa::kRatio128) return make_plan_r128(p);
  const Tuning& tu = tuning();
  Plan pl{};
  const int64_t W = int64_t{p.coff} * p.head_dim;
  pl.global_table = p.S > csa::kMaxLdsSegments;
  pl.off_bytes = pl.global_table ? align_up(uint64_t(p.S + 1) * 4, 256) : 0;

  // forward: one lane per (output row, chunk of C columns), grid-stride
  {
    const int C = choose_cols(p.head_dim, tu.fwd_cols);
    const int64_t G = p.head_dim / C;     // chunks of a row
    const int64_t Gp = pow2_ceil(G);      // lanes of a row
    const int64_t lanes = p.N * Gp;
    int64_t wgs = (lanes + csa::kFwdThreads - 1) / csa::kFwdThreads;
    // grid cap (measured on the 8192-token packs): 3 workgroups per CU at
    // ratio 4; ratio 2 windows hold half the bytes and want 4
    const int64_t cap = tu.fwd_max_wgs ? tu.fwd_max_wgs : (p.ratio >= 4 ? 768 : 1024);
    if (wgs > cap) wgs = cap;
    if (Gp > csa::kFwdThreads) wgs = align_up(wgs, Gp / csa::kFwdThreads);  // lanes % Gp == 0
    pl.fwd.grid = static_cast<uint32_t>(wgs);
    pl.fwd.threads = csa::kFwdThreads;
    pl.fwd.cols = C;
    pl.fwd.pad = Gp != G || C == 1;
    pl.fwd.uniform = tu.uniform && Gp >= 64;
    pl.fwd.prefetch = (pl.fwd.uniform && !pl.fwd.pad) ? tu.fwd_prefetch : 2;
    pl.fwd_log2_chunks = log2i(Gp);
    pl.fwd_chunks = static_cast<uint32_t>(G);
    const uint64_t table_words = pl.global_table ? 0 : 2 * (csa::kFwdThreads / 64) + 2 * uint64_t(p.S + 1);
    pl.fwd.lds_bytes = table_words * 4;
    pl.ws_fwd = pl.global_table ? kHeaderBytes + pl.off_bytes : 0;
  }
  // backward
  {
    const int C = choose_cols(p.head_dim, tu.bwd_cols);
    const int64_t G = p.head_dim / C;     // chunks of a row
    const int64_t Gp = pow2_ceil(G);      // lanes of a row
    const bool pad = Gp != G || C == 1;
    // 4 columns per lane need more than 128 VGPRs: at most 512 threads;
    // padded rows use 256-thread workgroups
    const int NT = pad ? 256 : (C == 4 && tu.bwd_threads > 512) ? 512 : tu.bwd_threads;
    // column slice per workgroup: at least 128 bytes of a half-row per wave
    // row (whole cache lines), at most the whole row and the workgroup
    int64_t CS = tu.bwd_slice_bytes / (2 * C);
    if (CS < 64 / C) CS = 64 / C;
    if (CS > Gp) CS = Gp;
    if (CS > NT) CS = NT;
    CS = pow2_floor(CS);  // the kernels take log2(CS): slices, partial rows and lanes must agree
    const int64_t slices = Gp / CS;
    const int64_t lanes = p.N * Gp;
    int64_t main = (lanes + NT - 1) / NT;
    // grid cap (measured on the 8192-token packs): one workgroup per CU at
    // ratio 4; ratio 2 windows hold half the bytes and want 2
    const int64_t cap = tu.bwd_max_wgs ? tu.bwd_max_wgs : (p.ratio >= 4 ? 256 : 512);
    if (main > cap) main = cap;
    main = align_up(main, slices);  // whole slices
    // zero-fill workgroups for rows of segments shorter than ratio and rows
    // past cu[S]: at most total_tokens - total_comp*ratio rows qualify
    const int64_t spare_rows = p.T - p.N * p.ratio;
    int64_t zero = 0;
    if (spare_rows > 0) {
      const int64_t bytes = spare_rows * W * 2 * 2;
      zero = (bytes + int64_t{NT} * 16 * 8 - 1) / (int64_t{NT} * 16 * 8);
      if (zero < 1) zero = 1;
      if (zero > 256) zero = 256;
    }
    if (main + zero == 0) zero = 1;  // someone must write the validity flag
    pl.bwd.grid = static_cast<uint32_t>(main + zero);
    pl.bwd.threads = NT;
    pl.bwd.cols = C;
    pl.bwd.pad = pad;
    pl.bwd.uniform = tu.uniform && CS >= 64;
    pl.bwd.prefetch = (pl.bwd.uniform && NT <= 512 && !pad) ? tu.bwd_prefetch : 2;
    pl.bwd_log2_chunks = log2i(Gp);
    pl.bwd_chunks = static_cast<uint32_t>(G);
    pl.bwd_log2_slice = log2i(CS);
    pl.bwd_main_wgs = static_cast<uint32_t>(main);
    pl.partial_rows = static_cast<uint32_t>(main / slices);
    // the dAPE staging follows the table and is read 16 bytes at a time:
    // keep it 16-byte aligned
    pl.lds_table_words =
        pl.global_table ? 0 : static_cast<uint32_t>(align_up(2 * (NT / 64) + 2 * uint64_t(p.S + 1), 4));
    const uint64_t red_floats = uint64_t(NT) * p.coff * p.ratio * C;  // dAPE staging: every thread's sums
    pl.bwd.lds_bytes = (uint64_t(pl.lds_table_words) + red_floats) * 4;
    pl.partial_offset = kHeaderBytes + pl.off_bytes;
    const uint64_t nblk = (uint64_t(p.ratio) * W + csa::kPartBlock - 1) / csa::kPartBlock;
    pl.ws_bwd = pl.partial_offset + align_up(nblk * pl.partial_rows * csa::kPartBlock * 4, 256);
  }
  return pl;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

csa_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(CSA_STATUS_INVALID_VALUE, "%s is null", name);
  if (!aligned16(p)) return fail(CSA_STATUS_INVALID_VALUE, "%s is not 16-byte aligned", name);
  return CSA_STATUS_SUCCESS;
}

// Host copy of cu_seqlens (optional): must describe the same pack as the
// problem; checked here so the kernels can trust it.
csa_status_t check_host_cu(const Problem& p, const int32_t* cu_host) {
  if (!cu_host) return CSA_STATUS_SUCCESS;
  if (cu_host[0] != 0) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens_host[0] must be 0");
  int64_t n = 0;
  for (int32_t s = 0; s < p.S; ++s) {
    const int64_t L = int64_t{cu_host[s + 1]} - cu_host[s];
    if (L < 0) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens_host decreases at %d", s);
    n += L / p.ratio;
  }
  if (cu_host[p.S] > p.T) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens_host[S] exceeds total_tokens");
  if (n != p.N)
    return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens_host gives %lld output rows, total_comp is %lld", (long long)n,
                (long long)p.N);
  return CSA_STATUS_SUCCESS;
}

csa::SegParams seg_params(const Problem& p, const Plan& pl, const int32_t* cu, const int32_t* cu_host, void* ws) {
  csa::SegParams sp{};
  sp.cu = cu;
  sp.T_cap = p.T;
  sp.N = p.N;
  sp.S = p.S;
  sp.table = csa::kTableLds;
  if (pl.global_table) {
    sp.table = csa::kTableGlobal;
    sp.g_flag = reinterpret_cast<const int32_t*>(ws);
    sp.g_off = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + kHeaderBytes);
  } else if (cu_host && p.S <= csa::kArgSegments) {
    sp.table = csa::kTableArgs;
    int32_t off = 0;
    for (int32_t s = 0; s <= p.S; ++s) {
      sp.arg_cu[s] = cu_host[s];
      sp.arg_off[s] = off;
      if (s < p.S) off += (cu_host[s + 1] - cu_host[s]) / p.ratio;
    }
  }
  return sp;
}

csa_status_t after_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CSA_STATUS_LAUNCH_FAILED, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

csa_status_t launch_scan_if_needed(const Problem& p, const Plan& pl, const int32_t* cu, void* ws,
                                   hipStream_t stream) {
  if (!pl.global_table) return CSA_STATUS_SUCCESS;
  const csa::SegParams sp = seg_params(p, pl, cu, nullptr, ws);
  int32_t* flag = reinterpret_cast<int32_t*>(ws);
  int32_t* off = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kHeaderBytes);
  if (!csa::launch_seg_scan(p.ratio, sp, off, flag, stream))
    return fail(CSA_STATUS_NOT_SUPPORTED, "no scan kernel for ratio %d", p.ratio);
  return after_launch("segment scan");
}

// Validation of the backward's tensors (shared by the backward entry points).
csa_status_t check_bwd_io(const Problem& pr, const void* kv, const void* score, const float* ape,
                          const int32_t* cu, const void* dout, const void* dkv, const void* dscore) {
  csa_status_t st;
  if (pr.T > 0) {
    if ((st = check_ptr(dkv, "dkv")) || (st = check_ptr(dscore, "dscore"))) return st;
  }
  if (pr.N > 0) {
    if ((st = check_ptr(kv, "kv")) || (st = check_ptr(score, "score")) || (st = check_ptr(ape, "ape")) ||
        (st = check_ptr(dout, "dout")))
      return st;
  }
  // the backward always launches (it must zero its outputs), so cu is read
  if (!cu) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens is null");
  if (reinterpret_cast<uintptr_t>(cu) & 3u) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens is not 4-byte aligned");
  return CSA_STATUS_SUCCESS;
}

// Validation shared by the backward entry points with a caller workspace.
csa_status_t check_bwd_args(const Problem& pr, const Plan& pl, const void* kv, const void* score,
                            const float* ape, const int32_t* cu, const void* dout, const void* dkv,
                            const void* dscore, const void* workspace, size_t workspace_bytes) {
  csa_status_t st;
  if ((st = check_bwd_io(pr, kv, score, ape, cu, dout, dkv, dscore))) return st;
  if (workspace_bytes < pl.ws_bwd)
    return fail(CSA_STATUS_WORKSPACE_TOO_SMALL, "backward needs %llu workspace bytes, got %llu",
                (unsigned long long)pl.ws_bwd, (unsigned long long)workspace_bytes);
  if ((st = check_ptr(workspace, "workspace"))) return st;
  return CSA_STATUS_SUCCESS;
}

csa_status_t launch_bwd_grads(const Problem& pr, const Plan& pl, const void* kv, const void* score,
                              const float* ape, const int32_t* cu, const int32_t* cu_host, const void* dout,
                              void* dkv, void* dscore, void* workspace, hipStream_t stream) {
  csa_status_t st = launch_scan_if_needed(pr, pl, cu, workspace, stream);
  if (st) return st;
  if (pr.ratio == csa::kRatio128) {
    csa::Bwd128Params bp{};
    bp.seg = seg_params(pr, pl, cu, cu_host, workspace);
    bp.kv = static_cast<const uint16_t*>(kv);
    bp.score = static_cast<const uint16_t*>(score);
    bp.ape = ape;
    bp.dout = static_cast<const uint16_t*>(dout);
    bp.dkv = static_cast<uint16_t*>(dkv);
    bp.dscore = static_cast<uint16_t*>(dscore);
    bp.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.partial_offset);
    bp.ws_flag = reinterpret_cast<int32_t*>(workspace);
    bp.io_bytes = static_cast<uint32_t>(pr.T * pr.coff * pr.head_dim * 2);
    bp.head_dim = pr.head_dim;
    bp.nslices = pl.nslices;
    bp.main_wgs = pl.bwd_main_wgs;
    bp.partial_rows = pl.partial_rows;
    bp.lds_table_words = pl.lds_table_words;
#ifdef CSA_DEBUG_OWNERSHIP
    bp.own_dkv = g_own_dkv;
    bp.own_dsc = g_own_dsc;
#endif
    if (!csa::launch_bwd128(pr.coff, bp, pl.bwd.grid, pl.bwd.lds_bytes, stream))
      return fail(CSA_STATUS_NOT_SUPPORTED, "no ratio-128 backward kernel for this configuration");
    return after_launch("backward");
  }
  csa::BwdParams bp{};
  bp.seg = seg_params(pr, pl, cu, cu_host, workspace);
  bp.kv = static_cast<const uint16_t*>(kv);
  bp.score = static_cast<const uint16_t*>(score);
  bp.ape = ape;
  bp.dout = static_cast<const uint16_t*>(dout);
  bp.dkv = static_cast<uint16_t*>(dkv);
  bp.dscore = static_cast<uint16_t*>(dscore);
  bp.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.partial_offset);
  bp.ws_flag = reinterpret_cast<int32_t*>(workspace);
  bp.io_bytes = static_cast<uint32_t>(pr.T * pr.coff * pr.head_dim * 2);
  bp.head_dim = pr.head_dim;
  bp.log2_chunks = pl.bwd_log2_chunks;
  bp.chunks = pl.bwd_chunks;
  bp.log2_slice = pl.bwd_log2_slice;
  bp.main_wgs = pl.bwd_main_wgs;
  bp.partial_rows = pl.partial_rows;
  bp.lds_table_words = pl.lds_table_words;
#ifdef CSA_DEBUG_OWNERSHIP
  bp.own_dkv = g_own_dkv;
  bp.own_dsc = g_own_dsc;
#endif
  if (!csa::launch_bwd(pr.ratio, pr.coff, bp, pl.bwd, stream))
    return fail(CSA_STATUS_NOT_SUPPORTED, "no backward kernel for this configuration");
  return after_launch("backward");
}

csa_status_t launch_reduce(const Problem& pr, const Plan& pl, float* dape, void* workspace, hipStream_t stream) {
  csa::ReduceParams rp{};
  rp.partials = reinterpret_cast<const float*>(static_cast<char*>(workspace) + pl.partial_offset);
  rp.dape = dape;
  rp.ws_flag = reinterpret_cast<const int32_t*>(workspace);
  rp.rows = pl.partial_rows;
  rp.cols = static_cast<uint32_t>(pr.ratio * pr.coff * pr.head_dim);
  csa::launch_dape_reduce(rp, stream);
  return after_launch("dAPE reduce");
}

}  // namespace

extern "C" {

const char* csa_status_string(csa_status_t status) {
  switch (status) {
    case CSA_STATUS_SUCCESS: return "CSA_STATUS_SUCCESS";
    case CSA_STATUS_INVALID_VALUE: return "CSA_STATUS_INVALID_VALUE";
    case CSA_STATUS_NOT_SUPPORTED: return "CSA_STATUS_NOT_SUPPORTED";
    case CSA_STATUS_WORKSPACE_TOO_SMALL: return "CSA_STATUS_WORKSPACE_TOO_SMALL";
    case CSA_STATUS_LAUNCH_FAILED: return "CSA_STATUS_LAUNCH_FAILED";
    case CSA_STATUS_DEVICE_ERROR: return "CSA_STATUS_DEVICE_ERROR";
  }
  return "CSA_STATUS_UNKNOWN";
}

const char* csa_last_error(void) { return g_err.c_str(); }

int32_t csa_version(void) { return 100; }

csa_status_t csa_compressor_total_comp(const int32_t* cu, int32_t S, int32_t ratio, int64_t* total_comp) {
  if (!cu || !total_comp) return fail(CSA_STATUS_INVALID_VALUE, "null pointer");
  if (S < 0 || ratio < 1) return fail(CSA_STATUS_INVALID_VALUE, "num_segments < 0 or ratio < 1");
  if (cu[0] != 0) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens[0] must be 0");
  int64_t n = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t L = int64_t{cu[s + 1]} - cu[s];
    if (L < 0) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens decreases at %d", s);
    n += L / ratio;
  }
  *total_comp = n;
  return ok();
}

csa_status_t csa_compressor_check_support(int32_t ratio, int32_t coff, int32_t head_dim, int32_t S,
                                          int64_t total_tokens, int64_t total_comp) {
  return check_problem(Problem{ratio, coff, head_dim, S, total_tokens, total_comp});
}

csa_status_t csa_compressor_fwd_workspace_size(int32_t ratio, int32_t coff, int32_t head_dim, int32_t S,
                                               int64_t total_tokens, int64_t total_comp, size_t* bytes) {
  if (!bytes) return fail(CSA_STATUS_INVALID_VALUE, "bytes is null");
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  const csa_status_t st = check_problem(pr);
  if (st) return st;
  *bytes = make_plan(pr).ws_fwd;
  return ok();
}

csa_status_t csa_compressor_bwd_workspace_size(int32_t ratio, int32_t coff, int32_t head_dim, int32_t S,
                                               int64_t total_tokens, int64_t total_comp, size_t* bytes) {
  if (!bytes) return fail(CSA_STATUS_INVALID_VALUE, "bytes is null");
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  const csa_status_t st = check_problem(pr);
  if (st) return st;
  *bytes = make_plan(pr).ws_bwd;
  return ok();
}

csa_status_t csa_compressor_fwd(const void* kv, const void* score, const float* ape, const int32_t* cu,
                                const int32_t* cu_host, int32_t S, int64_t total_tokens, int64_t total_comp,
                                int32_t ratio, int32_t coff, int32_t head_dim, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  csa_status_t st = check_problem(pr);
  if (st) return st;
  if ((st = check_host_cu(pr, cu_host))) return st;
  if (pr.N == 0) return ok();  // no output rows: nothing to do
  if ((st = check_ptr(kv, "kv")) || (st = check_ptr(score, "score")) || (st = check_ptr(ape, "ape")) ||
      (st = check_ptr(out, "out")))
    return st;
  if (!cu) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens is null");
  if (reinterpret_cast<uintptr_t>(cu) & 3u) return fail(CSA_STATUS_INVALID_VALUE, "cu_seqlens is not 4-byte aligned");
  const Plan pl = make_plan(pr);
  if (workspace_bytes < pl.ws_fwd)
    return fail(CSA_STATUS_WORKSPACE_TOO_SMALL, "forward needs %llu workspace bytes, got %llu",
                (unsigned long long)pl.ws_fwd, (unsigned long long)workspace_bytes);
  if (pl.ws_fwd > 0 && (st = check_ptr(workspace, "workspace"))) return st;

  if ((st = launch_scan_if_needed(pr, pl, cu, workspace, stream))) return st;
  if (ratio == csa::kRatio128) {
    csa::Fwd128Params fp{};
    fp.seg = seg_params(pr, pl, cu, cu_host, workspace);
    fp.kv = static_cast<const uint16_t*>(kv);
    fp.score = static_cast<const uint16_t*>(score);
    fp.ape = ape;
    fp.out = static_cast<uint16_t*>(out);
    fp.io_bytes = static_cast<uint32_t>(pr.T * pr.coff * pr.head_dim * 2);
    fp.head_dim = head_dim;
    fp.nslices = pl.nslices;
    fp.lds_table_words = pl.fwd_lds_table_words;
    if (!csa::launch_fwd128(coff, fp, pl.fwd.grid, pl.fwd.lds_bytes, stream))
      return fail(CSA_STATUS_NOT_SUPPORTED, "no ratio-128 forward kernel for this configuration");
    return after_launch("forward");
  }
  csa::FwdParams fp{};
  fp.seg = seg_params(pr, pl, cu, cu_host, workspace);
  fp.kv = static_cast<const uint16_t*>(kv);
  fp.score = static_cast<const uint16_t*>(score);
  fp.ape = ape;
  fp.out = static_cast<uint16_t*>(out);
  fp.io_bytes = static_cast<uint32_t>(pr.T * pr.coff * pr.head_dim * 2);
  fp.head_dim = head_dim;
  fp.log2_chunks = pl.fwd_log2_chunks;
  fp.chunks = pl.fwd_chunks;
  if (!csa::launch_fwd(ratio, coff, fp, pl.fwd, stream))
    return fail(CSA_STATUS_NOT_SUPPORTED, "no forward kernel for this configuration");
  return after_launch("forward");
}

csa_status_t csa_compressor_bwd_grads(const void* kv, const void* score, const float* ape, const int32_t* cu,
                                      const int32_t* cu_host, int32_t S, int64_t total_tokens, int64_t total_comp,
                                      int32_t ratio, int32_t coff, int32_t head_dim, const void* dout, void* dkv,
                                      void* dscore, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  csa_status_t st = check_problem(pr);
  if (st) return st;
  if ((st = check_host_cu(pr, cu_host))) return st;
  const Plan pl = make_plan(pr);
  if ((st = check_bwd_args(pr, pl, kv, score, ape, cu, dout, dkv, dscore, workspace, workspace_bytes))) return st;
  return launch_bwd_grads(pr, pl, kv, score, ape, cu, cu_host, dout, dkv, dscore, workspace, stream);
}

csa_status_t csa_compressor_bwd_dape_reduce(int32_t ratio, int32_t coff, int32_t head_dim, int32_t S,
                                            int64_t total_tokens, int64_t total_comp, float* dape,
                                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  csa_status_t st = check_problem(pr);
  if (st) return st;
  const Plan pl = make_plan(pr);
  if ((st = check_ptr(dape, "dape"))) return st;
  if (workspace_bytes < pl.ws_bwd)
    return fail(CSA_STATUS_WORKSPACE_TOO_SMALL, "backward needs %llu workspace bytes, got %llu",
                (unsigned long long)pl.ws_bwd, (unsigned long long)workspace_bytes);
  if ((st = check_ptr(workspace, "workspace"))) return st;
  return launch_reduce(pr, pl, dape, workspace, stream);
}

csa_status_t csa_compressor_bwd(const void* kv, const void* score, const float* ape, const int32_t* cu,
                                const int32_t* cu_host, int32_t S, int64_t total_tokens, int64_t total_comp,
                                int32_t ratio, int32_t coff, int32_t head_dim, const void* dout, void* dkv,
                                void* dscore, float* dape, int32_t deterministic, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  (void)deterministic;  // dAPE is always reduced in a fixed order
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  csa_status_t st = check_problem(pr);
  if (st) return st;
  if ((st = check_host_cu(pr, cu_host))) return st;
  const Plan pl = make_plan(pr);
  if ((st = check_bwd_args(pr, pl, kv, score, ape, cu, dout, dkv, dscore, workspace, workspace_bytes))) return st;
  if ((st = check_ptr(dape, "dape"))) return st;
  if ((st = launch_bwd_grads(pr, pl, kv, score, ape, cu, cu_host, dout, dkv, dscore, workspace, stream))) return st;
  return launch_reduce(pr, pl, dape, workspace, stream);
}

csa_status_t csa_compressor_bwd_noalloc(const void* kv, const void* score, const float* ape, const int32_t* cu,
                                        const int32_t* cu_host, int32_t S, int64_t total_tokens,
                                        int64_t total_comp, int32_t ratio, int32_t coff, int32_t head_dim,
                                        const void* dout, void* dkv, void* dscore, float* dape,
                                        int32_t deterministic, hipStream_t stream) {
  (void)deterministic;  // dAPE is always reduced in a fixed order
  const Problem pr{ratio, coff, head_dim, S, total_tokens, total_comp};
  csa_status_t st = check_problem(pr);
  if (st) return st;
  if ((st = check_host_cu(pr, cu_host))) return st;
  const Plan pl = make_plan(pr);
  if (pl.ws_bwd > csa::kNoAllocScratchBytes)
    return fail(CSA_STATUS_WORKSPACE_TOO_SMALL,
                "this problem needs %llu bytes of scratch; the allocation-free backward holds %llu per GPU "
                "(use csa_compressor_bwd with a workspace)",
                (unsigned long long)pl.ws_bwd, (unsigned long long)csa::kNoAllocScratchBytes);
  if ((st = check_bwd_io(pr, kv, score, ape, cu, dout, dkv, dscore))) return st;
  if ((st = check_ptr(dape, "dape"))) return st;
  void* ws = nullptr;
  const hipError_t e = csa::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(CSA_STATUS_DEVICE_ERROR, "library scratch of the current device not found: %s", hipGetErrorString(e));
  if ((st = launch_bwd_grads(pr, pl, kv, score, ape, cu, cu_host, dout, dkv, dscore, ws, stream))) return st;
  return launch_reduce(pr, pl, dape, ws, stream);
}

#ifdef CSA_DEBUG_OWNERSHIP
// Debug build only (libcsa_debug.so): device arrays of one uint32 per dkv /
// dscore element (total_tokens * coff * head_dim each, zeroed by the caller)
// that every later backward store adds 1 to; NULL, NULL switches counting
// off.  Not part of the ABI of libcsa.so.
csa_status_t csa_debug_ownership_counters(uint32_t* dkv_counts, uint32_t* dscore_counts) {
  g_own_dkv = dkv_counts;
  g_own_dsc = dscore_counts;
  return ok();
}
#endif

}  // extern "C"
