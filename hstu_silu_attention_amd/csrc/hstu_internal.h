// Internal interface between the host planner (hstu_abi.hip) and the gfx950
// kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// One user of the batch, as the kernels see it (32 bytes).
//  uoff/n:  new history rows uoff..uoff+n-1 of the packed row space
//  coff/c:  candidate rows Nu+coff..Nu+coff+c-1 of the packed row space
//  m:       cached history length (positions 0..m-1 live in the cache)
//  key_row: row of key 0 in the key/value source (slot cache: slot*capacity;
//           no cache: uoff, i.e. the user's first history row of the vqk buffer);
//           paged cache: the first entry of the user's row of the page table
struct UserRec {
  int32_t uoff, n, coff, c, m, key_row, pad0, pad1;
};

// Attention work item (32 bytes), everything a workgroup needs to start: one load.
//  hk:      (head << 1) | is_candidate_tile
//  q0, nq:  the tile's first query within the user's history (or candidate) rows and
//           its query count (<= the kernel's query-block size; 0: no work)
//  m:       the user's cached history length
//  rbase:   packed row of the tile's first query
//  key_end: keys [0, key_end) are visible to the tile
//  key_row: row of key 0 in the key/value source
//
// The items are grouped into kXcds bins, one per XCD, and laid out per workgroup:
// workgroups are dealt to the XCDs round-robin, so workgroup w runs on XCD w % kXcds
// and takes item w, which the planner fills from bin w % kXcds (position w / kXcds).
// All items of one (user, head) share a bin, so that user's keys and values stay in
// one L2.
constexpr int kXcds = 8;

struct AttnItem {
  int32_t hk, q0, nq, m, rbase, key_end, key_row, pad;
};

// Compact attention work item (8 bytes) as the host planner writes it: user -1 for no
// work, else code = (query block << 8) | (head << 1) | is_candidate. The plan kernel
// expands it into an AttnItem.
struct ItemCode {
  int32_t user, code;
};

struct PlanArgs {
  const UserRec* users;
  int32_t B, Nu, T;
  int2* row_info;        // [T] {user, position}
  const ItemCode* codes; // [grid]
  AttnItem* items;       // [grid] out
  int32_t grid, bm;      // attention workgroups; query rows per work item
};

// Host -> device transfer through kernel arguments: `words` 32-bit words (at most
// kUploadWords) copied to dst. Kernel arguments are captured by value when the launch
// is enqueued, so the host source can be reused at once, nothing is allocated and the
// host never waits for the device.
constexpr int kUploadWords = 896;
struct UploadArgs {
  uint32_t* dst;
  int32_t words, pad;
  uint32_t w[kUploadWords];
};

// Workspace buffers of one layer (rows in the packed order: history rows of every
// user, then candidate rows), each padded to a multiple of kRowPad rows; rows T..
// are never written and only ever feed discarded GEMM output rows.
//  xn   [T_pad][D]   normalised layer input, the float32 projection's A operand (the
//                    bfloat16 projection normalises inside: no buffer)
//  cs   [L][4D]      float32 column sums of each layer's W1 (bfloat16 only)
//  st   [T][D/128]   float2 {mean, sum of squared deviations from that mean} of each
//                    layer-input row over each 128-column group, in float32 (bfloat16
//                    only): written by the previous layer's output GEMM (the first
//                    layer's by a row pass)
//  vqk  [T_pad][3D]  V | Q | K after SiLU and position bias
//  aout [T_pad][3D]  U | O | U*O: the output GEMM's A operand. The projection writes
//                    U and the attention O; the float32 attention also writes the
//                    gate U*O, the bfloat16 output GEMM forms it from U and O while
//                    staging (those columns stay unused)
constexpr int kRowPad = 256;

// Normalised layer input Xn = (X - mean) / sqrt(var + eps), per row over D.
struct NormArgs {
  const void* x_lo;      // rows [0, Nu)
  const void* x_hi;      // rows [Nu, T)
  int32_t Nu, T, D;
  void* xn;              // [T_pad][D] out
};

constexpr float kNormEps = 1e-6f;

// Column sums cs[l][n] = sum_k W1_l[n][k] (float32) of every layer's projection weight,
// which is stored [4D][D] (output feature n in row n).
struct ColsumArgs {
  const void* const* w;  // [L] device pointers to the layers' W1
  int32_t L, D;
  float* cs;             // [L][4D] out
};

struct UvqkArgs {
  const void* xn;        // [T_pad][D] normalised rows (float32 path)
  const void* x_lo;      // layer input rows [0, Nu) (bfloat16 path, normalised inside)
  const void* x_hi;      // layer input rows [Nu, T)
  const float* cs;       // [4D] column sums of this layer's W1 (bfloat16 path)
  const float2* st;      // [T][D/128] row statistics of the layer input (bfloat16 path)
  int32_t Nu, T, D;
  const void* w;         // [4D][D]
  const void* pos;       // [max_len][3D], or nullptr (no absolute position bias)
  const int2* row_info;
  const UserRec* users;
  void* vqk;             // [T_pad][3D] out: V, Q, K (rows < T written)
  void* aout;            // [T_pad][3D] out: U into columns [0, D)
  void* cache_k;         // this layer's [slots][cap][D] or [pages][kPageRows][D], or nullptr
  void* cache_v;
  const int32_t* pages;  // paged cache: the page table (device), else nullptr
  int32_t npages;        // paged cache: pages of the pool; an id outside [0, npages) is skipped
};

// Rows of one page of a paged key/value cache: user row p lives in page
// table[key_row + p / kPageRows], row p % kPageRows.
constexpr int kPageRows = 64;

struct AttnArgs {
  const AttnItem* items; // [grid], item w for workgroup w
  int32_t Nu, D;
  float inv;             // 1 / max_len
  const void* vqk;       // [T_pad][3D]: Q, and the candidates' own K, V
  const void* kbase;     // key row r of user b is kbase + (key_row_b + r) * ld (contiguous), or
  const void* vbase;     // kbase + (pages[key_row_b + r / 64] * 64 + r % 64) * ld (paged)
  const int32_t* pages;  // paged cache: the page table (device), else nullptr
  int32_t npages;        // paged cache: pages of the pool (reads outside it give zeros)
  int64_t ld;
  void* aout;            // [T_pad][3D]: writes O (float32 also reads U, writes U*O)
  const void* rel;       // this layer's relative bias [H][max_len] (float32 for both dtypes:
                         // the bfloat16 path reads a widened copy), or nullptr
  int32_t max_len;
};

struct OutArgs {
  const void* aout;      // [T_pad][3D] A operand [U | O | U*O] (bfloat16: U | O read)
  const void* w;         // [D][3D]
  const void* x_lo;      // residual rows [0, Nu)
  const void* x_hi;      // residual rows [Nu, T)
  void* y_lo;            // output rows [0, Nu)
  void* y_hi;            // output rows [Nu, T)
  float2* st;            // [T][D/128] out: statistics of the output rows (or nullptr)
  int32_t Nu, T, D;
};

// Query rows per attention work item for a dtype.
int attn_block_rows(int dtype);

// History packing: the output is `chunks` 16-byte chunks, `cpr` per row.
struct PackArgs {
  const void* ctx;
  const void* act;
  void* out;
  int32_t chunks, cpr;
  bool interleave, bf16;
};

// Candidate scoring head: `layers` affine layers over [rows][D] candidate rows, ReLU
// between them; the last has `outcomes` outputs, each passed through the sigmoid.
constexpr int kMaxHeadLayers = 8, kMaxHeadWidth = 512, kMaxOutcomes = 16;
struct ScoreArgs {
  const void* x;
  float* prob;
  int32_t rows, D, layers, outcomes;
  const void* w[kMaxHeadLayers];      // [width][in] row-major
  const void* b[kMaxHeadLayers];      // [width]
  int32_t width[kMaxHeadLayers];      // output features of each layer (the last: outcomes)
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_upload(const UploadArgs& a, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_score(int dtype, const ScoreArgs& a, hipStream_t s);
hipError_t launch_norm(int dtype, const NormArgs& a, hipStream_t s);
hipError_t launch_colsum(const ColsumArgs& a, hipStream_t s);   // bfloat16 weights
// st[row][g] of the rows [0, Nu) of x_lo and [Nu, T) of x_hi (bfloat16)
hipError_t launch_rowstats(const void* x_lo, const void* x_hi, int Nu, int T, int D, float2* st, hipStream_t s);
hipError_t launch_uvqk(int dtype, const UvqkArgs& a, hipStream_t s);
// grid = kXcds * (longest bin)
hipError_t launch_attn(int dtype, int dh, const AttnArgs& a, int grid, hipStream_t s);
hipError_t launch_transpose(int esize, const void* src, void* dst, int rows, int cols, hipStream_t s);
// dst[i] = float(src[i]) for bfloat16 src, i < n (n < 2^31)
hipError_t launch_widen_bf16(const void* src, float* dst, int64_t n, hipStream_t s);
// Up to kTransposeList matrices of one shape [rows][cols], each to its own destination
// [cols][rows], in one launch.
constexpr int kTransposeList = 16;
struct TransposeList {
  const void* src[kTransposeList];
  void* dst[kTransposeList];
  int32_t rows, cols, count;
};
hipError_t launch_transpose_list(int esize, const TransposeList& t, hipStream_t s);
hipError_t launch_out(int dtype, const OutArgs& a, hipStream_t s);

}  // namespace hstu
