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

enum Epilogue { kEpiY = 0, kEpiArgmax = 1 };

// Rows up to kSmallMaxRows run the small-m kernels (64-channel tiles); more
// rows, up to kRowsPerLaunch per launch, the large-m kernel (128-channel
// tiles). Larger m is split into launches of kRowsPerLaunch rows.
constexpr int kSmallMaxRows = 64;
constexpr int kRowsPerLaunch = 192;

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
  void* y;
  int ytype;
  uint4* xf;              // x rearranged into MFMA B fragments (m >= 16)
  float* part;            // [2G][M][tile channels] split-tile partial sums
  uint32_t* tile_cnt;     // [P] arrival counters, zero between calls
  unsigned long long* keys;  // argmax keys: 8 copies x 256 rows x 16 u64 (one line per row), zero between calls
  uint32_t* done;         // [1] finished-workgroup counter, zero between calls
  int32_t* idx;
  float* maxval;
};

struct GemmPlan {
  int G, U, P;
  int nq;  // strips per tile of the small-m MFMA kernel (2 or 4)
  size_t ws_bytes;
  size_t off_cnt, off_part, off_keys, off_done, off_xf;
};

// Plan of one launch (m <= kRowsPerLaunch).
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int num_cu);

// qpass: read only the 8-bit view of the records (low nibbles at their
// midpoint); escapes are restored as in the exact pass.
hipError_t launch_gemm(const GemmParams& p, int epi, bool qpass, hipStream_t s);

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
