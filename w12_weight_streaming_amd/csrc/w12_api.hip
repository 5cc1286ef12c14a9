// extern "C" entry points of libw12 (declared in include/w12.h).
//
// Every call validates its arguments on the host and returns W12_EINVAL or
// W12_ENOSPC before launching anything (the refusal-before-running style of
// the poot-llm docs, "What is refused"), then enqueues its kernels on the
// caller's stream. Nothing here allocates memory.
#include <atomic>

#include "../../include/w12.h"
#include "w12_internal.h"

namespace {

constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxRows = 512;

bool shape_ok(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || n % 32 != 0 || k % 256 != 0 || k > kMaxK) return false;
  // escape offsets are u32: the weight count must fit
  return n <= (int64_t(0xFFFFFFFF) / k);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool matrix_ok(const w12_matrix* w) {
  return w && shape_ok(w->n, w->k) && w->records && w->e_top && w->esc_off && w->esc &&
         aligned(w->records, 16) && aligned(w->e_top, 4) && aligned(w->esc_off, 4) &&
         aligned(w->esc, 4);
}

w12::MatrixArgs args_of(const w12_matrix* w) {
  w12::MatrixArgs a;
  a.rec = w->records;
  a.e_top = w->e_top;
  a.esc_off = w->esc_off;
  a.esc = w->esc;
  a.n = w->n;
  a.k = w->k;
  a.nb = w->n * w->k / 1024;
  return a;
}

// Compute-unit count of the current device, cached per device id.
int num_cu() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

w12_status st(hipError_t e) { return e == hipSuccess ? W12_OK : W12_EHIP; }

// Workspace of a call: the largest of its launches' plans (rows are split
// into launches of at most w12::kRowsPerLaunch).
size_t gemm_ws_bytes(int64_t n, int64_t k, int64_t m, int cu) {
  size_t need = 0;
  for (int64_t m0 = 0; m0 < m; m0 += w12::kRowsPerLaunch) {
    const int64_t mc = m - m0 < w12::kRowsPerLaunch ? m - m0 : w12::kRowsPerLaunch;
    const size_t b = w12::plan_gemm(n, k, mc, cu).ws_bytes;
    if (b > need) need = b;
  }
  return need;
}

w12_status run_gemm(const w12_matrix* w, const uint16_t* x, int64_t m, void* y, int ytype,
                    int32_t* idx, float* maxval, void* ws, size_t ws_bytes, hipStream_t s,
                    int epi, bool qpass) {
  const int cu = num_cu();
  if (cu <= 0) return W12_EHIP;
  if (!ws) return W12_EINVAL;
  if (ws_bytes < gemm_ws_bytes(w->n, w->k, m, cu)) return W12_ENOSPC;
  char* base = static_cast<char*>(ws);
  const size_t y_row = (size_t)w->n * (ytype == W12_Y_F32 ? 4 : 2);
  for (int64_t m0 = 0; m0 < m; m0 += w12::kRowsPerLaunch) {
    const int64_t mc = m - m0 < w12::kRowsPerLaunch ? m - m0 : w12::kRowsPerLaunch;
    const w12::GemmPlan pl = w12::plan_gemm(w->n, w->k, mc, cu);
    w12::GemmParams p{};
    p.w = args_of(w);
    p.x = x + m0 * w->k;
    p.M = (int)mc;
    p.N = (int)w->n;
    p.K = (int)w->k;
    p.RK = (int)(w->k / 256);
    p.S = (int)(w->n / 32);
    p.P = pl.P;
    p.U = pl.U;
    p.G = pl.G;
    p.nq = pl.nq;
    p.xdirect = pl.xdirect;
    p.y = y ? static_cast<void*>(static_cast<char*>(y) + m0 * y_row) : nullptr;
    p.ytype = ytype;
    p.part = reinterpret_cast<float*>(base + pl.off_part);
    p.xf = reinterpret_cast<uint4*>(base + pl.off_xf);
    p.tile_cnt = reinterpret_cast<uint32_t*>(base + pl.off_cnt);
    p.keys = reinterpret_cast<unsigned long long*>(base + pl.off_keys);
    p.done = reinterpret_cast<uint32_t*>(base + pl.off_done);
    p.idx = idx ? idx + m0 : nullptr;
    p.maxval = maxval ? maxval + m0 : nullptr;
    const w12_status r = st(w12::launch_gemm(p, epi, qpass, s));
    if (r != W12_OK) return r;
  }
  return W12_OK;
}

// Workspace of the certified head. What must be zero between calls sits at
// the same offsets for every shape, so one workspace serves calls of any
// shape: the rescoring's keys, done counter and per-row counts first, then
// the INT8 pass's GEMM workspace (its own counters at its start; its
// argmax-key region holds the rows' lower bounds); what every call writes
// before it reads follows: row norms, then the upper bounds per 4-row group
// and row.
struct CertLayout {
  w12::GemmPlan pl;
  size_t off_keys2, off_done2, off_list_count, off_counts, off_xnorm, off_gemm, off_u4, off_list, total;
};
CertLayout cert_layout(int64_t n, int64_t k, int64_t m, int cu) {
  CertLayout L{};
  L.pl = w12::plan_gemm(n, k, m, cu);
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  L.off_keys2 = 0;
  L.off_done2 = w12::kKeyRegionBytes;
  L.off_list_count = L.off_done2 + 128;  // its own cache line
  L.off_counts = L.off_done2 + 256;
  L.off_xnorm = L.off_counts + 256;
  L.off_gemm = L.off_xnorm + 256;
  // the INT8 pass runs the MFMA kernel for every m, so its x fragments need
  // ceil(m / 32) tiles even below kMfmaMinRows rows (where plan_gemm reserves none)
  const size_t xf_end = L.pl.off_xf + (size_t)((m + 31) / 32) * 32 * (size_t)k * 2;
  L.off_u4 = up(L.off_gemm + (L.pl.ws_bytes > xf_end ? L.pl.ws_bytes : xf_end));
  L.off_list = up(L.off_u4 + (size_t)(n / 4) * w12::kCertMaxRows * 4);
  L.total = L.off_list + (size_t)(n / 4) * w12::kCertMaxRows * 8;
  return L;
}

w12_status gemm_entry(const w12_matrix* w, const uint16_t* x, int64_t m, void* y, int ytype,
                      void* ws, size_t ws_bytes, hipStream_t stream, bool qpass) {
  if (!matrix_ok(w) || !x || !y || m < 1 || m > kMaxRows) return W12_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16)) return W12_EINVAL;
  if (ytype != W12_Y_F32 && ytype != W12_Y_BF16) return W12_EINVAL;
  return run_gemm(w, x, m, y, ytype, nullptr, nullptr, ws, ws_bytes, stream, w12::kEpiY, qpass);
}

w12_status head_entry(const w12_matrix* head, const uint16_t* x, int64_t m, int32_t* idx,
                      float* maxval, void* ws, size_t ws_bytes, hipStream_t stream, bool qpass) {
  if (!matrix_ok(head) || !x || !idx || m < 1 || m > kMaxRows) return W12_EINVAL;
  if (!aligned(x, 16)) return W12_EINVAL;
  return run_gemm(head, x, m, nullptr, 0, idx, maxval, ws, ws_bytes, stream, w12::kEpiArgmax, qpass);
}

}  // namespace

extern "C" {

const char* w12_strerror(int status) {
  switch (status) {
    case W12_OK: return "W12_OK";
    case W12_EINVAL: return "W12_EINVAL: invalid argument";
    case W12_ENOSPC: return "W12_ENOSPC: workspace too small";
    case W12_EHIP: return "W12_EHIP: HIP runtime or launch error";
    case W12_ECORRUPT: return "W12_ECORRUPT: weights do not restore bit-for-bit (refused)";
    default: return "W12: unknown status";
  }
}

int w12_abi_version(void) { return 1; }

int64_t w12_num_blocks(int64_t n, int64_t k) {
  if (!shape_ok(n, k)) return -1;
  return n * k / 1024;
}

w12_status w12_pack_plan(const uint16_t* w, int64_t n, int64_t k, uint8_t* e_top,
                         uint32_t* esc_off, hipStream_t stream) {
  if (!w || !e_top || !esc_off || !shape_ok(n, k) || !aligned(w, 16)) return W12_EINVAL;
  return st(w12::launch_pack_plan(w, n, k, e_top, esc_off, stream));
}

w12_status w12_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top,
                    const uint32_t* esc_off, uint8_t* records, uint32_t* esc,
                    int64_t esc_capacity, hipStream_t stream) {
  if (!w || !e_top || !esc_off || !records || !shape_ok(n, k) || esc_capacity < 0)
    return W12_EINVAL;
  if (!aligned(w, 16) || !aligned(records, 16)) return W12_EINVAL;
  if (esc_capacity > 0 && !esc) return W12_EINVAL;
  return st(w12::launch_pack(w, n, k, e_top, esc_off, records, esc, esc_capacity, stream));
}

w12_status w12_decode(const w12_matrix* w, uint16_t* out, hipStream_t stream) {
  if (!matrix_ok(w) || !out || !aligned(out, 16)) return W12_EINVAL;
  return st(w12::launch_decode(args_of(w), out, stream));
}

w12_status w12_check(const w12_matrix* w, const uint16_t* ref, unsigned long long* mismatches,
                     hipStream_t stream) {
  if (!matrix_ok(w) || !ref || !mismatches || !aligned(ref, 16)) return W12_EINVAL;
  return st(w12::launch_check(args_of(w), ref, mismatches, stream));
}

w12_status w12_gemm_workspace(int64_t n, int64_t k, int64_t m, size_t* bytes) {
  if (!bytes || !shape_ok(n, k) || m < 1 || m > kMaxRows) return W12_EINVAL;
  const int cu = num_cu();
  if (cu <= 0) return W12_EHIP;
  *bytes = gemm_ws_bytes(n, k, m, cu);
  return W12_OK;
}


w12_status w12_gemm(const w12_matrix* w, const uint16_t* x, int64_t m, void* y, int ytype,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return gemm_entry(w, x, m, y, ytype, ws, ws_bytes, stream, false);
}

w12_status w12_gemm_qpass(const w12_matrix* w, const uint16_t* x, int64_t m, void* y, int ytype,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  return gemm_entry(w, x, m, y, ytype, ws, ws_bytes, stream, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------- no-allocation GEMM
//
// w12_gemm_noalloc runs w12_gemm's kernels with their workspace in `scratch`,
// a file-scope device array: one copy per device, held until the process
// ends. In host code the array's name is not a device address; the address
// each device gives for it is looked up once per device, with that device
// current, and only that pointer is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[W12_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Zero-fill of the scratch array at set-up: the workspace's arrival counters
// and argmax keys must start at zero (every completed call leaves them at
// zero again). A kernel rather than hipMemsetAsync, so that a set-up that
// happens inside stream capture records a kernel node.
__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
  std::atomic<int> state{0};  // 0 not set up, 1 setting up, 2 ready, 3 failed
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

// The scratch array's device address on the current device (nullptr on
// failure). The first caller on a device looks it up and enqueues the clear
// on its stream; callers racing with it wait until it is done.
void* scratch_ptr(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  int st_ = slot.state.load(std::memory_order_acquire);
  if (st_ == 2) return slot.ptr;
  if (st_ == 3) return nullptr;
  int expect = 0;
  if (slot.state.compare_exchange_strong(expect, 1, std::memory_order_acq_rel)) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p) {
      hipLaunchKernelGGL(scratch_clear_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p),
                         (size_t)W12_NOALLOC_SCRATCH_BYTES / 16);
      e = hipGetLastError();
    }
    slot.ptr = (e == hipSuccess) ? p : nullptr;
    slot.state.store(e == hipSuccess && p ? 2 : 3, std::memory_order_release);
    return slot.ptr;
  }
  while ((st_ = slot.state.load(std::memory_order_acquire)) == 1) {
  }
  return st_ == 2 ? slot.ptr : nullptr;
}

}  // namespace

extern "C" {

w12_status w12_gemm_noalloc(const w12_matrix* w, const uint16_t* x, int64_t m, void* y, int ytype,
                            hipStream_t stream) {
  if (!matrix_ok(w) || !x || !y || m < 1 || m > kMaxRows) return W12_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16)) return W12_EINVAL;
  if (ytype != W12_Y_F32 && ytype != W12_Y_BF16) return W12_EINVAL;
  const int cu = num_cu();
  if (cu <= 0) return W12_EHIP;
  if (gemm_ws_bytes(w->n, w->k, m, cu) > (size_t)W12_NOALLOC_SCRATCH_BYTES) return W12_ENOSPC;
  void* ws = scratch_ptr(stream);
  if (!ws) return W12_EHIP;
  return run_gemm(w, x, m, y, ytype, nullptr, nullptr, ws, W12_NOALLOC_SCRATCH_BYTES, stream,
                  w12::kEpiY, false);
}

w12_status w12_head_argmax_workspace(int64_t n, int64_t k, int64_t m, size_t* bytes) {
  return w12_gemm_workspace(n, k, m, bytes);
}

w12_status w12_head_argmax(const w12_matrix* head, const uint16_t* x, int64_t m, int32_t* idx,
                           float* maxval, void* ws, size_t ws_bytes, hipStream_t stream) {
  return head_entry(head, x, m, idx, maxval, ws, ws_bytes, stream, false);
}

w12_status w12_cert8_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top, int8_t* q,
                          uint8_t* qexp, float* cbound, hipStream_t stream) {
  if (!w || !e_top || !q || !qexp || !cbound || !shape_ok(n, k)) return W12_EINVAL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(cbound, 4)) return W12_EINVAL;
  return st(w12::launch_cert_pack(w, n, k, e_top, q, qexp, cbound, stream));
}

w12_status w12_head_argmax_certified_workspace(int64_t n, int64_t k, int64_t m, size_t* bytes) {
  if (!bytes || !shape_ok(n, k) || m < 1 || m > w12::kCertMaxRows) return W12_EINVAL;
  const int cu = num_cu();
  if (cu <= 0) return W12_EHIP;
  *bytes = cert_layout(n, k, m, cu).total;
  return W12_OK;
}

w12_status w12_head_argmax_certified(const w12_matrix* head, const w12_cert8* cert, const uint16_t* x, int64_t m,
                                     int32_t* idx, float* maxval, int32_t* rescored, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (!matrix_ok(head) || !cert || !x || !idx || !ws || m < 1 || m > w12::kCertMaxRows) return W12_EINVAL;
  if (cert->n != head->n || cert->k != head->k || !cert->q || !cert->qexp || !cert->cbound) return W12_EINVAL;
  if (!aligned(cert->q, 16) || !aligned(cert->qexp, 4) || !aligned(cert->cbound, 16) || !aligned(x, 16) ||
      !aligned(ws, 256))
    return W12_EINVAL;
  const int cu = num_cu();
  if (cu <= 0) return W12_EHIP;
  const CertLayout L = cert_layout(head->n, head->k, m, cu);
  if (w12::plan_slice_channels(L.pl, head->k) > w12::kCertCbFloats) return W12_EINVAL;
  if (ws_bytes < L.total) return W12_ENOSPC;
  char* base = static_cast<char*>(ws);
  w12::GemmParams p{};
  p.w = args_of(head);
  p.x = x;
  p.M = (int)m;
  p.N = (int)head->n;
  p.K = (int)head->k;
  p.RK = (int)(head->k / 256);
  p.S = (int)(head->n / 32);
  p.P = L.pl.P;
  p.U = L.pl.U;
  p.G = L.pl.G;
  p.nq = L.pl.nq;
  p.xdirect = L.pl.xdirect;
  char* gbase = base + L.off_gemm;
  p.part = reinterpret_cast<float*>(gbase + L.pl.off_part);
  p.xf = reinterpret_cast<uint4*>(gbase + L.pl.off_xf);
  p.tile_cnt = reinterpret_cast<uint32_t*>(gbase + L.pl.off_cnt);
  p.keys = reinterpret_cast<unsigned long long*>(gbase + L.pl.off_keys);
  p.done = reinterpret_cast<uint32_t*>(gbase + L.pl.off_done);
  p.cq = cert->q;
  p.cexp = cert->qexp;
  p.cbound = cert->cbound;
  p.xnorm = reinterpret_cast<float*>(base + L.off_xnorm);
  p.u4 = reinterpret_cast<float*>(base + L.off_u4);
  w12_status r = st(w12::launch_cert_pass(p, stream));
  if (r != W12_OK) return r;
  w12::CertRescoreArgs a{};
  a.w = p.w;
  a.x = x;
  a.M = (int)m;
  a.K = (int)head->k;
  a.u4 = p.u4;
  a.lb_keys = p.keys;
  a.keys = reinterpret_cast<unsigned long long*>(base + L.off_keys2);
  a.done = reinterpret_cast<uint32_t*>(base + L.off_done2);
  a.counts = reinterpret_cast<uint32_t*>(base + L.off_counts);
  a.list_count = reinterpret_cast<uint32_t*>(base + L.off_list_count);
  a.list = reinterpret_cast<uint2*>(base + L.off_list);
  a.idx = idx;
  a.maxval = maxval;
  a.rescored = rescored;
  return st(w12::launch_cert_rescore(a, 2 * cu, stream));
}

w12_status w12_head_argmax_qpass(const w12_matrix* head, const uint16_t* x, int64_t m, int32_t* idx,
                                 float* maxval, void* ws, size_t ws_bytes, hipStream_t stream) {
  return head_entry(head, x, m, idx, maxval, ws, ws_bytes, stream, true);
}

w12_status tree_accept(int32_t num_trees, const int32_t* node_off, int32_t total_nodes,
                       const int32_t* parent, const int32_t* token, const int32_t* argmax,
                       int32_t* accept_len, int32_t* path, int32_t* bonus, hipStream_t stream) {
  if (num_trees < 0 || total_nodes < 0) return W12_EINVAL;
  if (num_trees == 0) return W12_OK;
  if (!node_off || !accept_len || !bonus) return W12_EINVAL;
  if (total_nodes > 0 && (!parent || !token || !argmax || !path)) return W12_EINVAL;
  return st(w12::launch_tree_accept(num_trees, node_off, total_nodes, parent, token, argmax,
                                    accept_len, path, bonus, stream));
}

namespace {
// Limits of the tree builder's kernels: K, D <= 16 (4-bit ranks, 16-level
// rank paths); R <= 128 and budget - R <= 1023 (request and position fields
// of the 64-bit selection key); R (budget - R) <= 8192 (keys held in LDS).
bool tree_build_ok(int32_t R, int32_t D, int32_t K, int32_t budget) {
  if (R < 1 || R > 128 || D < 1 || D > 16 || K < 1 || K > 16) return false;
  if (budget < R || budget - R > 1023) return false;
  return (int64_t)R * (budget - R) <= 8192;
}
}  // namespace

w12_status w12_tree_build_workspace(int32_t num_req, int32_t budget, size_t* bytes) {
  if (!bytes || !tree_build_ok(num_req, 1, 1, budget)) return W12_EINVAL;
  *bytes = w12::tree_build_ws_bytes(num_req, budget);
  return W12_OK;
}

w12_status w12_tree_build(int32_t num_req, int32_t positions, int32_t k, const float* lp, const int32_t* tok,
                          const int32_t* depth, const int32_t* root, int32_t budget, void* ws,
                          size_t ws_bytes, int32_t* node_off, int32_t* parent, int32_t* token,
                          int32_t* node_depth, float* score, hipStream_t stream) {
  if (!tree_build_ok(num_req, positions, k, budget)) return W12_EINVAL;
  if (!lp || !tok || !depth || !root || !node_off || !parent || !token || !ws) return W12_EINVAL;
  if (!aligned(ws, 16) || !aligned(lp, 4)) return W12_EINVAL;
  if (ws_bytes < w12::tree_build_ws_bytes(num_req, budget)) return W12_ENOSPC;
  return st(w12::launch_tree_build(num_req, positions, k, lp, tok, depth, root, budget, ws, node_off, parent,
                                   token, node_depth, score, stream));
}

}  // extern "C"
