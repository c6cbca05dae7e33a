// csa_launch.h -- internal interface between the C ABI (csa_api.cpp) and the
// gfx950 kernels (csa_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

constexpr int kFwdThreads = 256;
// Packs with more segments than this build their offset table with a
// separate scan kernel into the workspace instead of in each workgroup's LDS.
constexpr int kMaxLdsSegments = 2048;
// Packs with at most this many segments whose host copy of cu_seqlens is
// given take cu and the block offsets as kernel arguments.
constexpr int kArgSegments = 32;

// dAPE partial rows are stored in column blocks of this many floats (one
// 128-byte line per partial row and block).
constexpr int kPartBlock = 32;

// Where the kernels find the segment table.
enum TableKind : int32_t {
  kTableLds = 0,     // built per workgroup in LDS from the device cu_seqlens
  kTableGlobal = 1,  // built in the workspace by seg_scan_kernel (large packs)
  kTableArgs = 2,    // passed in the kernel arguments (host copy, small packs)
};

struct SegParams {
  const int32_t* cu;      // device cu_seqlens [S + 1]
  const int32_t* g_off;   // offsets in the workspace (large packs) or null
  const int32_t* g_flag;  // validity flag in the workspace (large packs) or null
  int64_t T_cap;          // total_tokens (row capacity)
  int64_t N;              // total_comp as given by the caller
  int32_t S;
  int32_t table;          // TableKind
  int32_t arg_cu[kArgSegments + 1];   // kTableArgs: cu_seqlens
  int32_t arg_off[kArgSegments + 1];  // kTableArgs: output-block offsets
};

struct FwdParams {
  SegParams seg;
  const uint16_t* kv;
  const uint16_t* score;
  const float* ape;
  uint16_t* out;
  uint32_t io_bytes;      // total_tokens * coff * head_dim * 2
  uint32_t head_dim;
  uint32_t log2_chunks;   // log2(lanes per row): head_dim / cols rounded up to a power of two
  uint32_t chunks;        // head_dim / cols (chunks of a row; lanes past it are padding)
};

struct BwdParams {
  SegParams seg;
  const uint16_t* kv;
  const uint16_t* score;
  const float* ape;
  const uint16_t* dout;
  uint16_t* dkv;
  uint16_t* dscore;
  float* partials;        // column blocks [ceil(ratio*W/kPartBlock)][partial_rows][kPartBlock]
  int32_t* ws_flag;       // validity flag in the workspace
  uint32_t io_bytes;
  uint32_t head_dim;
  uint32_t log2_chunks;   // log2(lanes per row), as in FwdParams
  uint32_t chunks;        // head_dim / cols
  uint32_t log2_slice;    // log2(chunks per workgroup column slice)
  uint32_t main_wgs;      // workgroups [0, main_wgs) compute windows, the rest zero-fill
  uint32_t partial_rows;  // main_wgs / slices
  uint32_t lds_table_words;
  uint32_t* own_dkv;      // ownership counters, one per dkv / dscore element: every store
  uint32_t* own_dsc;      // adds 1 (builds with CSA_DEBUG_OWNERSHIP only; null otherwise)
};

// ratio = 128 (windows of 128 * coff rows): a workgroup owns a slice of
// kSlice128 columns (one per lane) and walks output rows; head_dim must be a
// multiple of kSlice128.  Forward: workgroups of 4 * coff waves (two per CU
// at coff 2, four at coff 1) compute a window in two halves of 64 * coff
// rows, staged in LDS: dynamic LDS = the segment table, two half-window
// stages (score and kv rows, bf16) and an exchange area of three floats per
// wave and column (wave maximum, wave Z, wave acc).  Backward: workgroups of
// kThreads128 threads, one per CU (grids capped at kCUs), each window copied
// into one of two static LDS buffers; kRed128Bytes is its dynamic LDS
// exchange area after the segment table (wave maxima, wave Z, wave acc).
constexpr int kRatio128 = 128;
constexpr int kSlice128 = 64;
constexpr int fwd128_threads(int coff) { return 4 * coff * 64; }
constexpr int fwd128_stage_bytes(int coff) { return 2 * (2 * 64 * coff * kSlice128 * 2); }
constexpr int fwd128_red_bytes(int coff) { return 3 * 4 * coff * kSlice128 * 4; }
constexpr int kThreads128 = 1024;
constexpr int kRed128Bytes = 3 * (kThreads128 / 64) * kSlice128 * 4;
constexpr int kCUs = 256;  // MI355X

struct Fwd128Params {
  SegParams seg;
  const uint16_t* kv;
  const uint16_t* score;
  const float* ape;
  uint16_t* out;
  uint32_t io_bytes;
  uint32_t head_dim;
  uint32_t nslices;       // head_dim / kSlice128
  uint32_t lds_table_words;
};

struct Bwd128Params {
  SegParams seg;
  const uint16_t* kv;
  const uint16_t* score;
  const float* ape;
  const uint16_t* dout;
  uint16_t* dkv;
  uint16_t* dscore;
  float* partials;        // column blocks [ceil(128*W/kPartBlock)][partial_rows][kPartBlock]
  int32_t* ws_flag;
  uint32_t io_bytes;
  uint32_t head_dim;
  uint32_t nslices;
  uint32_t main_wgs;      // = the grid: every workgroup computes windows, then zero-fills its share
  uint32_t partial_rows;  // main_wgs / nslices
  uint32_t lds_table_words;
  uint32_t* own_dkv;      // ownership counters as in BwdParams
  uint32_t* own_dsc;
};

struct ReduceParams {
  const float* partials;
  float* dape;
  const int32_t* ws_flag;
  uint32_t rows;
  uint32_t cols;          // ratio * coff * head_dim
};

struct LaunchShape {
  uint32_t grid;
  uint32_t threads;
  uint32_t cols;          // output columns per lane (1, 2 or 4)
  bool uniform;           // every wave works on one output row at a time
  bool pad;               // lanes per row rounded up past head_dim / cols (or cols == 1)
  uint32_t prefetch;      // windows in flight per lane (uniform path: 2, 3, 4)
  size_t lds_bytes;
};

bool launch_fwd(int ratio, int coff, const FwdParams& p, const LaunchShape& sh, hipStream_t st);
bool launch_bwd(int ratio, int coff, const BwdParams& p, const LaunchShape& sh, hipStream_t st);
void launch_dape_reduce(const ReduceParams& p, hipStream_t st);
bool launch_seg_scan(int ratio, const SegParams& sp, int32_t* off, int32_t* flag, hipStream_t st);
bool launch_fwd128(int coff, const Fwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st);
bool launch_bwd128(int coff, const Bwd128Params& p, uint32_t grid, size_t lds_bytes, hipStream_t st);

// Library-owned device scratch of the allocation-free backward: its size and
// the address of the current device's copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t{40} << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace csa
