// Host-side launch interface between the C ABI (w12_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

struct MatrixArgs {
  const uint8_t* rec;
  const uint8_t* e_top;
  const uint32_t* esc_off;
  const uint32_t* esc;
  int64_t n, k, nb;
};

enum Epilogue { kEpiY = 0, kEpiArgmax = 1, kEpiCert = 2 };

// Weight formats the small-m MFMA kernel streams: W12 records, or the
// certified head's INT8 copy (8 KB records laid out as W12's 8-bit-view
// plane, one scale code per 32-k block of a channel, W12's escapes).
enum Format { kFmtW12 = 0, kFmtCert8 = 1 };
constexpr int kCertRecBytes = 8192;
// floats of per-channel bound constants a workgroup of the INT8 pass keeps
// in LDS (the channels of its slice's tiles)
constexpr int kCertCbFloats = 4096;
// rows of the certified head (one MFMA path, at most two 32-row tiles)
constexpr int kCertMaxRows = 64;

// Rows up to kSmallMaxRows run the small-m kernels (64- or 128-channel
// tiles); more rows, up to kRowsPerLaunch per launch, the large-m kernel
// (128-channel tiles). Larger m is split into launches of kRowsPerLaunch rows.
constexpr int kSmallMaxRows = 64;
constexpr int kRowsPerLaunch = 192;
// Rows from which the small-m path multiplies on the matrix cores (one
// 32-row x tile, rows past m zero); fewer rows take the VALU dot products.
// Measured on Wgate|Wup 34816x5120: 56.5-56.8 us for every m in 5..16 on
// the matrix cores (x pre-pass included), against 67-98 us on the VALU path;
// 1-4 rows stay on the VALU path, which takes 52-56 us there.
constexpr int kMfmaMinRows = 5;

// Argmax keys in a workspace: kKeyCopies copies (workgroup b uses copy
// b % kKeyCopies, one per XCD) x kKeyRows rows x kKeyStride u64 (one
// 128-byte line per row). The certified head reads and clears its lower
// bounds in the same layout.
constexpr int kKeyCopies = 8;
constexpr int kKeyRows = 256;  // >= kRowsPerLaunch
constexpr int kKeyStride = 16;
constexpr size_t kKeyRegionBytes = size_t(8) * kKeyCopies * kKeyRows * kKeyStride;

// One verify GEMM (or LM head) launch. Work is split stream-K style: a unit
// is one record of a tile (2 strips of 32 channels for small m, 4 for large
// m), units run tile-major, and workgroup g owns units [g*U/G, (g+1)*U/G).
struct GemmParams {
  MatrixArgs w;
  const uint16_t* x;
  int M, N, K;
  int RK;  // records per strip = K / 256
  int S;   // strips = N / 32
  int P;   // tiles = ceil(S / strips per tile)
  int U;   // units = P * RK
  int G;   // workgroups
  int nq;  // strips per tile of the small-m MFMA kernel (from the plan)
  int xdirect;  // small-m MFMA kernel: x fragments straight from row-major x, no pre-pass (from the plan)
  void* y;
  int ytype;
  uint4* xf;              // x rearranged into MFMA B fragments (m >= kMfmaMinRows)
  float* part;            // [2G][M][tile channels] split-tile partial sums
  uint32_t* tile_cnt;     // [P] arrival counters, zero between calls
  unsigned long long* keys;  // argmax keys: 8 copies x 256 rows x 16 u64 (one line per row), zero between calls
  uint32_t* done;         // [1] finished-workgroup counter, zero between calls
  int32_t* idx;
  float* maxval;
  // certified head's INT8 pass (kEpiCert): the copy, the bound constants,
  // the row norms of x, and the upper bounds per 4-channel group and row
  const int8_t* cq;
  const uint8_t* cexp;
  const float* cbound;
  const float* xnorm;
  float* u4;  // [ceil(N / 4)][64]
};

// Certified head: the INT8 copy's pack, and the rescoring that follows the
// INT8 pass.
struct CertRescoreArgs {
  MatrixArgs w;            // the W12 head (records and escapes for the exact logits)
  const uint16_t* x;
  int M, K;
  const float* u4;         // [ceil(N / 4)][64] upper bounds
  unsigned long long* lb_keys;  // per-row lower bounds (argmax key layout), cleared at the end
  unsigned long long* keys;     // exact argmax keys (same layout), cleared at the end
  uint32_t* done;
  uint32_t* counts;        // [64] rescored vocabulary rows per input row, cleared at the end
  uint32_t* list_count;    // entries the selection listed, cleared at the end
  uint2* list;             // [N / 4 * 64] entries (group, row)
  int32_t* idx;
  float* maxval;
  int32_t* rescored;
};
hipError_t launch_cert_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top, int8_t* q,
                            uint8_t* code, float* cbound, hipStream_t s);
// the selection (groups whose upper bound reaches a row's lower bound) and
// the exact rescoring of the selected groups (rescore_grid workgroups)
hipError_t launch_cert_rescore(const CertRescoreArgs& a, int rescore_grid, hipStream_t s);

struct GemmPlan {
  int G, U, P;
  int nq;  // strips per tile of the small-m MFMA kernel (2 or 4)
  int xdirect;  // 1: the small-m MFMA kernel reads x row-major and the x pre-pass is skipped
  size_t ws_bytes;
  size_t off_cnt, off_part, off_keys, off_done, off_xf;
};

// Plan of one launch (m <= kRowsPerLaunch).
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int num_cu, int max_nq = 4);

// qpass: read only the 8-bit view of the records (low nibbles at their
// midpoint); escapes are restored as in the exact pass.
hipError_t launch_gemm(const GemmParams& p, int epi, bool qpass, hipStream_t s);

// The certified head's INT8 pass (m <= kCertMaxRows): x fragments and row
// norms, then the MFMA pass over the INT8 copy with the bound epilogue.
// p.xnorm and p.u4 point into the workspace.
hipError_t launch_cert_pass(const GemmParams& p, hipStream_t s);
// Largest number of channels one workgroup's slice covers in a plan (the
// INT8 pass keeps their bound constants in LDS).
int64_t plan_slice_channels(const GemmPlan& pl, int64_t k);

hipError_t launch_pack_plan(const uint16_t* w, int64_t n, int64_t k, uint8_t* e_top,
                            uint32_t* esc_off, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top,
                       const uint32_t* esc_off, uint8_t* rec, uint32_t* esc, int64_t cap,
                       hipStream_t s);
hipError_t launch_decode(const MatrixArgs& a, uint16_t* out, hipStream_t s);
hipError_t launch_check(const MatrixArgs& a, const uint16_t* ref, unsigned long long* mism,
                        hipStream_t s);
// Best-first draft trees under a shared row budget (tree_build.hip).
size_t tree_build_ws_bytes(int32_t num_req, int32_t budget);
hipError_t launch_tree_build(int32_t R, int32_t D, int32_t K, const float* lp, const int32_t* tok,
                             const int32_t* depth, const int32_t* roots, int32_t budget, void* ws,
                             int32_t* node_off, int32_t* parent, int32_t* token, int32_t* node_depth,
                             float* score, hipStream_t s);
hipError_t launch_tree_accept(int32_t num_trees, const int32_t* node_off, int32_t total,
                              const int32_t* parent, const int32_t* token, const int32_t* argmax,
                              int32_t* accept_len, int32_t* path, int32_t* bonus, hipStream_t s);

}  // namespace w12
