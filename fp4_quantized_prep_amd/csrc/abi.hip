// C ABI of libiqprep.so (declared and documented in include/iqprep.h).
//
// Every entry point validates its arguments on the host first; nothing that
// fails validation touches the device. Then it checks, once per device, that
// the current device is gfx950, and enqueues its kernel on the caller's stream.
#include <atomic>
#include <cstring>
#include <mutex>

#include "iqp_internal.h"
#include "iqprep.h"

// The allocation-free entry point's scratch: the split-K workspace for up to
// IQP_NOALLOC_MAX_HEADS heads, in static device storage (zero when the
// library's code is loaded on a device; every call leaves its counters at zero
// again). Each GPU holds its own copy until the process ends. Host code uses
// only the per-device address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) uint8_t scratch[iqp::splitk_workspace_bytes(IQP_NOALLOC_MAX_HEADS)];

namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet queried, 1 = gfx950, 2 = other architecture, 3 = query failed
std::atomic<int> g_arch_state[kMaxDevices];

int device_status() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return IQP_ERR_HIP;
  if (dev >= kMaxDevices) return IQP_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      st = 3;
    } else {
      st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? IQP_OK : (st == 2 ? IQP_ERR_UNSUPPORTED : IQP_ERR_HIP);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// the current device's address of scratch, looked up once per device (with
// that device current) and kept
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return IQP_ERR_HIP;
  if (dev >= kMaxDevices) return IQP_ERR_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return IQP_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = static_cast<uint8_t*>(ptr);
  return IQP_OK;
}

// Packed scale words: [M, nw] logically; K-major or MN-major strides only.
int check_scale_strides(int64_t M, int64_t nw, int64_t sm, int64_t sw) {
  if (sw == 1 && sm >= nw && sm >= 1) return IQP_OK;
  if (sm == 1 && sw >= M && sw >= 1) return IQP_OK;
  return IQP_ERR_INVALID;
}

int from_hip(hipError_t e) { return e == hipSuccess ? IQP_OK : IQP_ERR_HIP; }

// Shared argument checks of the fused call and its diagnostic twin.
int check_indexer_q_args(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_sm,
                         int64_t as_sw, const void* w, int64_t ldw, const uint8_t* w_scales,
                         int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                         const int64_t* positions, const float* cos_sin, int64_t max_pos,
                         const void* out0, const void* out1) {
  if (M < 0 || K < 0 || H < 0 || D < 0 || rope_dim < 0 || max_pos < 0) return IQP_ERR_INVALID;
  if (M == 0) return IQP_OK;
  if (!a || !a_scales || !w || !w_scales || !positions || !cos_sin || !out0 || !out1)
    return IQP_ERR_INVALID;
  if (K == 0 || H == 0 || max_pos == 0) return IQP_ERR_INVALID;
  if (lda < K || ldw < K) return IQP_ERR_INVALID;
  const int64_t nw = (K / 128 + 3) / 4;
  if (K % 128) return IQP_ERR_UNSUPPORTED;
  if (check_scale_strides(M, nw, as_sm, as_sw) != IQP_OK) return IQP_ERR_INVALID;
  if (D != 128 || rope_dim != 64) return IQP_ERR_UNSUPPORTED;
  if (!aligned(a, 16) || lda % 16 || !aligned(w, 16) || ldw % 16 || !aligned(a_scales, 4) ||
      !aligned(positions, 8) || !aligned(cos_sin, 16))
    return IQP_ERR_UNSUPPORTED;
  if ((int64_t)H * 128 > ((int64_t)1 << 31)) return IQP_ERR_UNSUPPORTED;
  // the kernel keeps a head's weight-scale bytes in one register (4 per lane)
  if (K / 128 > 256) return IQP_ERR_UNSUPPORTED;
  // the kernel addresses one 256-row tile (and its scale words) with 32-bit offsets
  if (lda >= ((int64_t)1 << 23) || ldw >= ((int64_t)1 << 23)) return IQP_ERR_UNSUPPORTED;
  if (as_sm >= ((int64_t)1 << 20) || nw * as_sw >= ((int64_t)1 << 28)) return IQP_ERR_UNSUPPORTED;
  return IQP_OK;
}

iqp::IndexerQArgs make_args(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_sm,
                            int64_t as_sw, const void* w, int64_t ldw, const uint8_t* w_scales,
                            int64_t M, int64_t K, int32_t H, const int64_t* positions,
                            const float* cos_sin, int64_t max_pos) {
  iqp::IndexerQArgs p{};
  p.a = static_cast<const uint8_t*>(a);
  p.lda = lda;
  p.a_scale_bytes = reinterpret_cast<const uint8_t*>(a_scales);
  p.as_sm = as_sm;
  p.as_sw = as_sw;
  p.w = static_cast<const uint8_t*>(w);
  p.ldw = ldw;
  p.w_scales = w_scales;
  p.M = M;
  p.nkb = (int32_t)(K / 128);
  p.H = H;
  p.positions = positions;
  p.cos_sin = cos_sin;
  p.max_pos = max_pos;
  return p;
}

// Checks of the one-launch call and its diagnostic twin (outputs: 16-byte
// aligned out0, 4-byte aligned out1); fills p on success (M == 0: IQP_OK,
// nothing filled).
int prep_bf16_args(const void* x, int64_t ldx, const void* w, int64_t ldw, const uint8_t* w_scales,
                   int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                   const int64_t* positions, const float* cos_sin, int64_t max_pos,
                   const void* out0, const void* out1, iqp::IndexerQArgs& p) {
  if (M < 0 || K < 0 || H < 0 || D < 0 || rope_dim < 0 || max_pos < 0) return IQP_ERR_INVALID;
  if (M == 0) return IQP_OK;
  if (!x || !w || !w_scales || !positions || !cos_sin || !out0 || !out1) return IQP_ERR_INVALID;
  if (K == 0 || H == 0 || max_pos == 0) return IQP_ERR_INVALID;
  if (ldx < K || ldw < K) return IQP_ERR_INVALID;
  if (K != 1536 || M > 256 || D != 128 || rope_dim != 64) return IQP_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || ldx % 8 || !aligned(w, 16) || ldw % 16 || !aligned(w_scales, 4) ||
      !aligned(positions, 8) || !aligned(cos_sin, 16) || !aligned(out0, 16) || !aligned(out1, 4))
    return IQP_ERR_UNSUPPORTED;
  if ((int64_t)H * 128 > ((int64_t)1 << 31) || H > 65535 || ldw >= ((int64_t)1 << 22))
    return IQP_ERR_UNSUPPORTED;
  const int st = device_status();
  if (st != IQP_OK) return st;
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.w = static_cast<const uint8_t*>(w);
  p.ldw = ldw;
  p.w_scales = w_scales;
  p.M = M;
  p.nkb = (int32_t)(K / 128);
  p.H = H;
  p.positions = positions;
  p.cos_sin = cos_sin;
  p.max_pos = max_pos;
  if (!iqp::indexer_q_small_bf16_supported(p)) return IQP_ERR_UNSUPPORTED;
  return IQP_OK;
}

}  // namespace

extern "C" {

int fp8_quant_1x128_ue8m0(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq,
                          int32_t* scales, int64_t s_stride_m, int64_t s_stride_w, void* stream) {
  if (M < 0 || K < 0) return IQP_ERR_INVALID;
  if (M == 0 || K == 0) return IQP_OK;
  if (!x || !q || !scales) return IQP_ERR_INVALID;
  if (ldx < K || ldq < K) return IQP_ERR_INVALID;
  if (K % 128) return IQP_ERR_UNSUPPORTED;
  if (check_scale_strides(M, (K / 128 + 3) / 4, s_stride_m, s_stride_w) != IQP_OK) return IQP_ERR_INVALID;
  if (!aligned(x, 16) || ldx % 8 || !aligned(q, 8) || ldq % 8 || !aligned(scales, 4))
    return IQP_ERR_UNSUPPORTED;
  if (K / 128 > 0x7FFFFFFF) return IQP_ERR_UNSUPPORTED;
  const int ds = device_status();
  if (ds != IQP_OK) return ds;
  return from_hip(iqp::launch_fp8_quant(static_cast<const uint16_t*>(x), M, K, ldx,
                                        static_cast<uint8_t*>(q), ldq, scales, s_stride_m,
                                        s_stride_w, static_cast<hipStream_t>(stream)));
}

int indexer_q_gemm_rope_fp4(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_stride_m,
                            int64_t as_stride_w, const void* w, int64_t ldw, const uint8_t* w_scales,
                            int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                            const int64_t* positions, const float* cos_sin, int64_t max_pos,
                            uint8_t* q_fp4, uint8_t* q_scales, void* stream) {
  return indexer_q_gemm_rope_fp4_ex(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M, K, H, D,
                                    rope_dim, positions, cos_sin, max_pos, q_fp4, q_scales, 0, stream);
}

int indexer_q_gemm_rope_fp4_ex(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_stride_m,
                               int64_t as_stride_w, const void* w, int64_t ldw, const uint8_t* w_scales,
                               int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                               const int64_t* positions, const float* cos_sin, int64_t max_pos,
                               uint8_t* q_fp4, uint8_t* q_scales, int32_t flags, void* stream) {
  if (flags & ~(IQP_ROPE_INTERLEAVED | IQP_FP4_SCALE_OCP_FLOOR | IQP_W_SCALES_PER_ROW)) return IQP_ERR_INVALID;
  int st = check_indexer_q_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M, K,
                                H, D, rope_dim, positions, cos_sin, max_pos, q_fp4, q_scales);
  if (st != IQP_OK || M == 0) return st;
  if (!aligned(q_fp4, 16) || !aligned(q_scales, 4)) return IQP_ERR_UNSUPPORTED;
  st = device_status();
  if (st != IQP_OK) return st;
  iqp::IndexerQArgs p = make_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M,
                                  K, H, positions, cos_sin, max_pos);
  p.q_fp4 = q_fp4;
  p.q_scales = q_scales;
  return from_hip(iqp::launch_indexer_q_variant(p, flags, static_cast<hipStream_t>(stream)));
}

int indexer_q_gemm_rope_fp4_lanes(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_stride_m,
                                  int64_t as_stride_w, const void* w, int64_t ldw, const uint8_t* w_scales,
                                  int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                  const int64_t* positions, const float* cos_sin, const float* cos_sin_lanes,
                                  int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, void* stream) {
  int st = check_indexer_q_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M, K,
                                H, D, rope_dim, positions, cos_sin, max_pos, q_fp4, q_scales);
  if (st != IQP_OK || M == 0) return st;
  if (!cos_sin_lanes) return IQP_ERR_INVALID;
  if (!aligned(q_fp4, 16) || !aligned(q_scales, 4) || !aligned(cos_sin_lanes, 16)) return IQP_ERR_UNSUPPORTED;
  st = device_status();
  if (st != IQP_OK) return st;
  iqp::IndexerQArgs p = make_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M,
                                  K, H, positions, cos_sin, max_pos);
  p.cos_sin_lanes = cos_sin_lanes;
  p.q_fp4 = q_fp4;
  p.q_scales = q_scales;
  return from_hip(iqp::launch_indexer_q(p, -1, static_cast<hipStream_t>(stream)));
}

int indexer_q_prep_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, const uint8_t* w_scales,
                        int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                        const int64_t* positions, const float* cos_sin, int64_t max_pos,
                        uint8_t* q_fp4, uint8_t* q_scales, void* stream) {
  return indexer_q_prep_bf16_ex(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos,
                                q_fp4, q_scales, 0, stream);
}

int indexer_q_prep_bf16_ex(const void* x, int64_t ldx, const void* w, int64_t ldw, const uint8_t* w_scales,
                           int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                           const int64_t* positions, const float* cos_sin, int64_t max_pos,
                           uint8_t* q_fp4, uint8_t* q_scales, int32_t flags, void* stream) {
  if (flags & ~(IQP_ROPE_INTERLEAVED | IQP_FP4_SCALE_OCP_FLOOR | IQP_W_SCALES_PER_ROW)) return IQP_ERR_INVALID;
  iqp::IndexerQArgs p{};
  const int st = prep_bf16_args(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos,
                                q_fp4, q_scales, p);
  if (st != IQP_OK || M == 0) return st;
  p.q_fp4 = q_fp4;
  p.q_scales = q_scales;
  return from_hip(iqp::launch_indexer_q_small_bf16_variant(p, flags, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// indexer_q_prep_bf16_with_quant, with the small-batch kernel split over K
// where a workspace is given: ws of ws_bytes, or (use_scratch) this device's
// scratch, looked up after every check has passed (null and false: not split)
int prep_with_quant(const void* x, int64_t ldx, const void* w, int64_t ldw, const uint8_t* w_scales, int64_t M,
                    int64_t K, int32_t H, int32_t D, int32_t rope_dim, const int64_t* positions,
                    const float* cos_sin, int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, const void* x2,
                    int64_t M2, int64_t K2, int64_t ldx2, void* q2, int64_t ldq2, int32_t* scales2,
                    int64_t s_stride_m2, int64_t s_stride_w2, uint8_t* ws, int64_t ws_bytes, bool use_scratch,
                    void* stream) {
  // the second matrix: fp8_quant_1x128_ue8m0's checks, at decode sizes
  if (M2 < 0 || K2 < 0) return IQP_ERR_INVALID;
  const bool side = M2 > 0 && K2 > 0;
  if (side) {
    if (!x2 || !q2 || !scales2) return IQP_ERR_INVALID;
    if (ldx2 < K2 || ldq2 < K2) return IQP_ERR_INVALID;
    if (K2 % 128) return IQP_ERR_UNSUPPORTED;
    if (check_scale_strides(M2, (K2 / 128 + 3) / 4, s_stride_m2, s_stride_w2) != IQP_OK) return IQP_ERR_INVALID;
    if (!aligned(x2, 16) || ldx2 % 8 || !aligned(q2, 8) || ldq2 % 8 || !aligned(scales2, 4))
      return IQP_ERR_UNSUPPORTED;
    if (M2 > 256 || K2 / 128 > 0x7FFFFFFF) return IQP_ERR_UNSUPPORTED;
  }
  iqp::IndexerQArgs p{};
  const int st = prep_bf16_args(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos,
                                q_fp4, q_scales, p);
  if (st != IQP_OK) return st;
  if (M == 0) {   // no tokens for the projection: the quantization alone
    if (!side) return IQP_OK;
    const int ds = device_status();
    if (ds != IQP_OK) return ds;
    return from_hip(iqp::launch_fp8_quant(static_cast<const uint16_t*>(x2), M2, K2, ldx2, static_cast<uint8_t*>(q2),
                                          ldq2, scales2, s_stride_m2, s_stride_w2, static_cast<hipStream_t>(stream)));
  }
  p.q_fp4 = q_fp4;
  p.q_scales = q_scales;
  if (use_scratch) {
    const int ss = scratch_address(&ws);
    if (ss != IQP_OK) return ss;
    ws_bytes = (int64_t)sizeof(scratch);
  }
  p.splitk_ws = ws;
  p.splitk_ws_bytes = ws_bytes;
  if (side) {
    p.side_x = static_cast<const uint16_t*>(x2);
    p.side_ldx = ldx2;
    p.side_q = static_cast<uint8_t*>(q2);
    p.side_ldq = ldq2;
    p.side_scales = scales2;
    p.side_sm = s_stride_m2;
    p.side_sw = s_stride_w2;
    p.side_nkb = (int32_t)(K2 / 128);
    p.side_nw = (p.side_nkb + 3) / 4;
    p.side_words = M2 * p.side_nw;
  }
  return from_hip(iqp::launch_indexer_q_small_bf16(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int indexer_q_prep_bf16_with_quant(const void* x, int64_t ldx, const void* w, int64_t ldw, const uint8_t* w_scales,
                                   int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                   const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                   uint8_t* q_fp4, uint8_t* q_scales, const void* x2, int64_t M2, int64_t K2,
                                   int64_t ldx2, void* q2, int64_t ldq2, int32_t* scales2, int64_t s_stride_m2,
                                   int64_t s_stride_w2, void* stream) {
  return prep_with_quant(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos, q_fp4,
                         q_scales, x2, M2, K2, ldx2, q2, ldq2, scales2, s_stride_m2, s_stride_w2, nullptr, 0, false,
                         stream);
}

int64_t indexer_q_workspace_bytes(int32_t H) { return H > 0 ? iqp::splitk_workspace_bytes(H) : 0; }

int indexer_q_prep_bf16_with_quant_ws(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const uint8_t* w_scales, int64_t M, int64_t K, int32_t H, int32_t D,
                                      int32_t rope_dim, const int64_t* positions, const float* cos_sin,
                                      int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, const void* x2,
                                      int64_t M2, int64_t K2, int64_t ldx2, void* q2, int64_t ldq2,
                                      int32_t* scales2, int64_t s_stride_m2, int64_t s_stride_w2,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
  if (!workspace || (H > 0 && workspace_bytes < iqp::splitk_workspace_bytes(H))) return IQP_ERR_INVALID;
  if (!aligned(workspace, 256)) return IQP_ERR_UNSUPPORTED;
  return prep_with_quant(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos, q_fp4,
                         q_scales, x2, M2, K2, ldx2, q2, ldq2, scales2, s_stride_m2, s_stride_w2,
                         static_cast<uint8_t*>(workspace), workspace_bytes, false, stream);
}

int indexer_q_prep_bf16_with_quant_noalloc(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                           const uint8_t* w_scales, int64_t M, int64_t K, int32_t H, int32_t D,
                                           int32_t rope_dim, const int64_t* positions, const float* cos_sin,
                                           int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, const void* x2,
                                           int64_t M2, int64_t K2, int64_t ldx2, void* q2, int64_t ldq2,
                                           int32_t* scales2, int64_t s_stride_m2, int64_t s_stride_w2,
                                           void* stream) {
  if (H > IQP_NOALLOC_MAX_HEADS) return IQP_ERR_UNSUPPORTED;   // more than the scratch holds
  return prep_with_quant(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos, q_fp4,
                         q_scales, x2, M2, K2, ldx2, q2, ldq2, scales2, s_stride_m2, s_stride_w2, nullptr, 0, true,
                         stream);
}

int iqp_debug_indexer_q_prep_bf16_f32(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const uint8_t* w_scales, int64_t M, int64_t K, int32_t H, int32_t D,
                                      int32_t rope_dim, const int64_t* positions, const float* cos_sin,
                                      int64_t max_pos, float* out, void* stream) {
  iqp::IndexerQArgs p{};
  const int st = prep_bf16_args(x, ldx, w, ldw, w_scales, M, K, H, D, rope_dim, positions, cos_sin, max_pos,
                                out, out, p);
  if (st != IQP_OK || M == 0) return st;
  p.dbg = out;
  return from_hip(iqp::launch_indexer_q_small_dump(p, static_cast<hipStream_t>(stream)));
}

int iqp_debug_indexer_q_f32(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_stride_m,
                            int64_t as_stride_w, const void* w, int64_t ldw, const uint8_t* w_scales,
                            int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                            const int64_t* positions, const float* cos_sin, int64_t max_pos,
                            float* out, int32_t stage, void* stream) {
  if (stage < 0 || stage > 3) return IQP_ERR_INVALID;
  int st = check_indexer_q_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M, K,
                                H, D, rope_dim, positions, cos_sin, max_pos, out, out);
  if (st != IQP_OK || M == 0) return st;
  if (!aligned(out, 16)) return IQP_ERR_UNSUPPORTED;
  st = device_status();
  if (st != IQP_OK) return st;
  iqp::IndexerQArgs p = make_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M,
                                  K, H, positions, cos_sin, max_pos);
  p.dbg = out;
  if (stage == 3) return from_hip(iqp::launch_indexer_q_gemm_dump(p, static_cast<hipStream_t>(stream)));
  return from_hip(iqp::launch_indexer_q(p, stage, static_cast<hipStream_t>(stream)));
}

int iqp_debug_indexer_q_clock(const void* a, int64_t lda, const int32_t* a_scales, int64_t as_stride_m,
                              int64_t as_stride_w, const void* w, int64_t ldw, const uint8_t* w_scales,
                              int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                              const int64_t* positions, const float* cos_sin, const float* cos_sin_lanes,
                              int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, uint64_t* stamps,
                              int64_t stamp_capacity, int64_t* n_workgroups, void* stream) {
  if (!n_workgroups) return IQP_ERR_INVALID;
  *n_workgroups = 0;
  if (stamp_capacity < 0) return IQP_ERR_INVALID;
  int st = check_indexer_q_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M, K,
                                H, D, rope_dim, positions, cos_sin, max_pos, q_fp4, q_scales);
  if (st != IQP_OK) return st;
  if (M == 0) return IQP_ERR_UNSUPPORTED;
  if (!stamps) return IQP_ERR_INVALID;
  if (!aligned(q_fp4, 16) || !aligned(q_scales, 4) || !aligned(stamps, 16) || !aligned(cos_sin_lanes, 16))
    return IQP_ERR_UNSUPPORTED;
  st = device_status();
  if (st != IQP_OK) return st;
  iqp::IndexerQArgs p = make_args(a, lda, a_scales, as_stride_m, as_stride_w, w, ldw, w_scales, M,
                                  K, H, positions, cos_sin, max_pos);
  p.cos_sin_lanes = cos_sin_lanes;
  p.q_fp4 = q_fp4;
  p.q_scales = q_scales;
  p.dbg = reinterpret_cast<float*>(stamps);
  const hipError_t e = iqp::launch_indexer_q_clock(p, stamp_capacity, n_workgroups, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return IQP_ERR_UNSUPPORTED;
  if (e == hipErrorInvalidValue) return IQP_ERR_INVALID;
  return from_hip(e);
}

int iqp_device_clock_rates(int64_t* wall_clock_hz, int64_t* peak_shader_clock_hz) {
  if (!wall_clock_hz || !peak_shader_clock_hz) return IQP_ERR_INVALID;
  int dev = 0, wall_khz = 0, sclk_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(&sclk_khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return IQP_ERR_HIP;
  *wall_clock_hz = (int64_t)wall_khz * 1000;
  *peak_shader_clock_hz = (int64_t)sclk_khz * 1000;
  return IQP_OK;
}

int indexer_q_rope_hadamard_fp4(const void* q, int64_t ldq, int64_t M, int32_t H, int32_t D,
                                int32_t rope_dim, const int64_t* positions, const float* cos_sin,
                                int64_t max_pos, uint8_t* q_fp4, uint8_t* q_scales, int32_t flags,
                                void* stream) {
  if (M < 0 || H < 0 || D < 0 || rope_dim < 0 || max_pos < 0) return IQP_ERR_INVALID;
  if (flags & ~(IQP_ROPE_INTERLEAVED | IQP_FP4_SCALE_OCP_FLOOR)) return IQP_ERR_INVALID;
  if (M == 0) return IQP_OK;
  if (!q || !positions || !cos_sin || !q_fp4 || !q_scales) return IQP_ERR_INVALID;
  if (H == 0 || max_pos == 0) return IQP_ERR_INVALID;
  if (D != 128 || rope_dim != 64) return IQP_ERR_UNSUPPORTED;
  if (ldq < (int64_t)H * D) return IQP_ERR_INVALID;
  if (!aligned(q, 16) || ldq % 8 || !aligned(positions, 8) || !aligned(cos_sin, 16) ||
      !aligned(q_fp4, 16) || !aligned(q_scales, 4))
    return IQP_ERR_UNSUPPORTED;
  if (M > 0x7FFFFFFF || H > 64 * 65535) return IQP_ERR_UNSUPPORTED;
  const int st = device_status();
  if (st != IQP_OK) return st;
  return from_hip(iqp::launch_indexer_q_epilogue(static_cast<const uint16_t*>(q), ldq, M, H, positions,
                                                 cos_sin, max_pos, q_fp4, q_scales,
                                                 (flags & IQP_ROPE_INTERLEAVED) != 0,
                                                 (flags & IQP_FP4_SCALE_OCP_FLOOR) != 0,
                                                 static_cast<hipStream_t>(stream)));
}

int fp8_quant_weight_128x128_ue8m0(const void* w, int64_t N, int64_t K, int64_t ldw, void* q, int64_t ldq,
                                   uint8_t* scales, int64_t ld_scales, void* stream) {
  if (N < 0 || K < 0) return IQP_ERR_INVALID;
  if (N == 0 || K == 0) return IQP_OK;
  if (!w || !q || !scales) return IQP_ERR_INVALID;
  if (ldw < K || ldq < K || ld_scales < (K + 127) / 128) return IQP_ERR_INVALID;
  if (N % 128 || K % 128) return IQP_ERR_UNSUPPORTED;
  if (!aligned(w, 16) || ldw % 8 || !aligned(q, 8) || ldq % 8) return IQP_ERR_UNSUPPORTED;
  if (N / 128 > 65535 || K / 128 > 0x7FFFFFFF) return IQP_ERR_UNSUPPORTED;
  const int st = device_status();
  if (st != IQP_OK) return st;
  return from_hip(iqp::launch_fp8_quant_weight(static_cast<const uint16_t*>(w), N, K, ldw, static_cast<uint8_t*>(q),
                                               ldq, scales, ld_scales, static_cast<hipStream_t>(stream)));
}

int iqp_rope_cos_sin_table(double theta, int64_t max_pos, int32_t rope_dim, float* cos_sin,
                           void* stream) {
  if (max_pos < 0 || rope_dim <= 0 || rope_dim % 2 || !(theta > 0.0)) return IQP_ERR_INVALID;
  if (max_pos == 0) return IQP_OK;
  if (!cos_sin) return IQP_ERR_INVALID;
  if (!aligned(cos_sin, 4)) return IQP_ERR_UNSUPPORTED;
  const int st = device_status();
  if (st != IQP_OK) return st;
  return from_hip(iqp::launch_rope_table(theta, max_pos, rope_dim, cos_sin,
                                         static_cast<hipStream_t>(stream)));
}

int iqp_rope_table_lanes(const float* cos_sin, int64_t max_pos, int32_t rope_dim, float* out, void* stream) {
  if (max_pos < 0 || rope_dim < 0) return IQP_ERR_INVALID;
  if (max_pos == 0) return IQP_OK;
  if (!cos_sin || !out) return IQP_ERR_INVALID;
  if (rope_dim != 64) return IQP_ERR_UNSUPPORTED;
  if (!aligned(cos_sin, 16) || !aligned(out, 16)) return IQP_ERR_UNSUPPORTED;
  const int st = device_status();
  if (st != IQP_OK) return st;
  return from_hip(iqp::launch_rope_table_lanes(cos_sin, max_pos, out, static_cast<hipStream_t>(stream)));
}

const char* iqp_status_string(int status) {
  switch (status) {
    case IQP_OK: return "IQP_OK";
    case IQP_ERR_INVALID: return "IQP_ERR_INVALID: invalid argument";
    case IQP_ERR_UNSUPPORTED: return "IQP_ERR_UNSUPPORTED: outside the kernel's contract";
    case IQP_ERR_HIP: return "IQP_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown iqprep status";
  }
}

int iqp_abi_version(void) { return IQP_ABI_VERSION; }

}  // extern "C"
