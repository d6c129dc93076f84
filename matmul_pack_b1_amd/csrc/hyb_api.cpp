// Host side of the C ABI: layout planning and argument checks.  Nothing here
// touches the device except the final kernel launch through hyb_internal.h,
// so every error path can be exercised without a GPU.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "hyb_internal.h"

namespace {

thread_local std::string g_last_error;

hyb_status fail(hyb_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hyb_status ok() {
  g_last_error.clear();
  return HYB_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool device_tile(int32_t b) { return b == 64 || b == 128 || b == 256; }

int elem_size(int32_t dt) { return dt == HYB_F32 ? 4 : 2; }

// Shape and type checks shared by hyb_plan and the layout validator.
hyb_status check_geometry(int64_t n, int64_t k, int32_t b1, int32_t b2, int32_t dtype,
                          int32_t meta) {
  if (dtype != HYB_F16 && dtype != HYB_BF16)
    return fail(HYB_ERR_DTYPE, "dtype %d is not HYB_F16 or HYB_BF16", dtype);
  if (meta != HYB_META_IDX2 && meta != HYB_META_MASK4 && meta != HYB_META_MASK8)
    return fail(HYB_ERR_INVALID_ARG, "meta %d is not HYB_META_IDX2, HYB_META_MASK4 or HYB_META_MASK8", meta);
  if (b1 <= 0 || b2 <= 0 || b1 % 16 != 0 || b2 % 64 != 0)
    return fail(HYB_ERR_SHAPE, "tile %dx%d: need b1 %% 16 == 0 and b2 %% 64 == 0", b1, b2);
  if (n < 0 || k < 0) return fail(HYB_ERR_SHAPE, "negative shape %lldx%lld", (long long)n, (long long)k);
  if (n % b1 != 0 || k % b2 != 0)
    return fail(HYB_ERR_SHAPE, "shape %lldx%lld is not a whole number of %dx%d tiles",
                (long long)n, (long long)k, b1, b2);
  // Keep every stream index inside int64 with room to spare.
  if (n > (int64_t(1) << 31) || k > (int64_t(1) << 31) || n * k > (int64_t(1) << 40))
    return fail(HYB_ERR_SHAPE, "shape %lldx%lld too large", (long long)n, (long long)k);
  return HYB_OK;
}

void fill_sizes(hyb_layout* L) {
  const int64_t tile = int64_t(L->b1) * L->b2;
  L->dense_bytes = L->n_dense * tile * 2;
  L->val_bytes = L->n_sparse * tile;
  L->meta_bytes = L->n_sparse * tile / 8;
  L->tidx_bytes = L->tiles_n * L->tiles_k * 4;
}

// Full consistency check of a caller-held layout (magic, version, sizes).
hyb_status check_layout(const hyb_layout* L, bool device_call) {
  if (!L) return fail(HYB_ERR_INVALID_ARG, "layout is NULL");
  if (L->magic != HYB_MAGIC || L->version != HYB_VERSION)
    return fail(HYB_ERR_FORMAT, "layout magic/version 0x%08x/%u, expected 0x%08x/%u", L->magic,
                L->version, HYB_MAGIC, HYB_VERSION);
  hyb_status st = check_geometry(L->n, L->k, L->b1, L->b2, L->dtype, L->meta);
  if (st != HYB_OK) return st;
  if (L->tiles_n != L->n / L->b1 || L->tiles_k != L->k / L->b2 || L->n_dense < 0 ||
      L->n_sparse < 0 || L->n_dense + L->n_sparse != L->tiles_n * L->tiles_k)
    return fail(HYB_ERR_FORMAT, "layout tile counts are inconsistent");
  hyb_layout ref = *L;
  fill_sizes(&ref);
  if (ref.dense_bytes != L->dense_bytes || ref.val_bytes != L->val_bytes ||
      ref.meta_bytes != L->meta_bytes || ref.tidx_bytes != L->tidx_bytes)
    return fail(HYB_ERR_FORMAT, "layout byte sizes are inconsistent");
  if (device_call && !(device_tile(L->b1) && device_tile(L->b2)))
    return fail(HYB_ERR_UNSUPPORTED, "device kernels need b1, b2 in {64, 128, 256}, got %dx%d",
                L->b1, L->b2);
  return HYB_OK;
}

hyb_status check_packed(const hyb_layout* L, const hyb_packed* P) {
  if (!P) return fail(HYB_ERR_INVALID_ARG, "packed streams descriptor is NULL");
  if (L->dense_bytes > 0 && (!P->dense || !aligned(P->dense, 16)))
    return fail(HYB_ERR_INVALID_ARG, "dense stream is NULL or not 16-byte aligned");
  if (L->val_bytes > 0 && (!P->val || !aligned(P->val, 16)))
    return fail(HYB_ERR_INVALID_ARG, "value stream is NULL or not 16-byte aligned");
  if (L->meta_bytes > 0 && (!P->meta || !aligned(P->meta, 16)))
    return fail(HYB_ERR_INVALID_ARG, "metadata stream is NULL or not 16-byte aligned");
  if (L->tidx_bytes > 0 && (!P->tidx || !aligned(P->tidx, 4)))
    return fail(HYB_ERR_INVALID_ARG, "tile index is NULL or not 4-byte aligned");
  return HYB_OK;
}

hyb_status check_matrix_arg(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* name) {
  // A negative stride is rejected even for an empty operand: kernels build
  // buffer ranges from rows * ld, which must never go negative.
  if (ld < 0) return fail(HYB_ERR_INVALID_ARG, "%s row stride %lld is negative", name, (long long)ld);
  if (rows == 0 || cols == 0) return HYB_OK;
  if (!p) return fail(HYB_ERR_INVALID_ARG, "%s is NULL", name);
  if (ld < cols) return fail(HYB_ERR_INVALID_ARG, "%s row stride %lld < %lld", name, (long long)ld, (long long)cols);
  if (!aligned(p, 16) || ld % 8 != 0)
    return fail(HYB_ERR_INVALID_ARG, "%s must be 16-byte aligned with a row stride multiple of 8", name);
  return HYB_OK;
}

hyb_status check_product(const hyb_layout* L, const hyb_packed* P, const void* x, int32_t m,
                         int64_t ldx, const void* y, int32_t y_dtype, int64_t ldy, int32_t max_m) {
  hyb_status st = check_layout(L, true);
  if (st != HYB_OK) return st;
  if (m < 0 || m > max_m) return fail(HYB_ERR_SHAPE, "m = %d outside [0, %d]", m, max_m);
  if (y_dtype != HYB_F32 && y_dtype != L->dtype)
    return fail(HYB_ERR_DTYPE, "y_dtype %d must be HYB_F32 or the weight dtype %d", y_dtype, L->dtype);
  if (m == 0) return HYB_OK;
  st = check_packed(L, P);
  if (st != HYB_OK) return st;
  st = check_matrix_arg(x, m, L->k, ldx, "x");
  if (st != HYB_OK) return st;
  if (L->n > 0) {
    if (!y) return fail(HYB_ERR_INVALID_ARG, "y is NULL");
    if (ldy < L->n) return fail(HYB_ERR_INVALID_ARG, "y row stride %lld < n = %lld", (long long)ldy, (long long)L->n);
    if (!aligned(y, elem_size(y_dtype))) return fail(HYB_ERR_INVALID_ARG, "y is not aligned to its element size");
  }
  return HYB_OK;
}

// Launch limits of the matrix-core kernels (m > 0, n > 0).
hyb_status check_mfma_limits(int32_t m, int64_t ldx) {
  if (ldx < 0) return fail(HYB_ERR_INVALID_ARG, "ldx %lld is negative", (long long)ldx);
  if (ldx * 2 * 256 >= (int64_t(1) << 31))
    return fail(HYB_ERR_UNSUPPORTED, "matrix-core kernel needs ldx < 4194304 elements");
  if ((int64_t(m) + 15) / 16 > 65535 * 8) return fail(HYB_ERR_UNSUPPORTED, "m = %d too large for one launch", m);
  return HYB_OK;
}

hyb_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HYB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Workspace of the split-K launches of hyb_gemm and hyb_gemm_lowrank, held
// by the library: one buffer of kSplitMaxBytes per (device, stream),
// allocated at the first split launch there and kept until the process
// ends.  Work on one stream runs in order, so its launches can share the
// buffer; launches on different streams get different buffers.  Nothing is
// allocated while the stream is being captured into a graph (HIP refuses
// that): such a launch runs unsplit unless the stream already holds a
// buffer.  Returns {nullptr, 0} when the product does not split or no
// buffer is available (the product then runs unsplit, on the same kernel).
std::pair<void*, size_t> stream_workspace(const hyb_layout& L, int m, void* stream) {
  if (hyb::gemm_route(L, m, hyb::device_cus()).kernel != hyb::kRouteSplit) return {nullptr, 0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return {nullptr, 0};
  static std::mutex mu;
  static std::map<std::pair<int, void*>, void*> held;
  std::lock_guard<std::mutex> lock(mu);
  void*& p = held[{dev, stream}];
  if (!p) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess ||
        cap != hipStreamCaptureStatusNone)
      return {nullptr, 0};
    if (hipMalloc(&p, hyb::kSplitMaxBytes) != hipSuccess) {
      p = nullptr;
      (void)hipGetLastError();
      return {nullptr, 0};
    }
  }
  return {p, hyb::kSplitMaxBytes};
}

}  // namespace

extern "C" {

int32_t hyb_abi_version(void) { return HYB_ABI_VERSION; }

const char* hyb_status_str(hyb_status s) {
  switch (s) {
    case HYB_OK: return "HYB_OK";
    case HYB_ERR_INVALID_ARG: return "HYB_ERR_INVALID_ARG";
    case HYB_ERR_SHAPE: return "HYB_ERR_SHAPE";
    case HYB_ERR_DTYPE: return "HYB_ERR_DTYPE";
    case HYB_ERR_UNSUPPORTED: return "HYB_ERR_UNSUPPORTED";
    case HYB_ERR_FORMAT: return "HYB_ERR_FORMAT";
    case HYB_ERR_HIP: return "HYB_ERR_HIP";
    default: return "HYB_ERR_UNKNOWN";
  }
}

const char* hyb_last_error(void) { return g_last_error.c_str(); }

hyb_status hyb_plan(int64_t n, int64_t k, int32_t b1, int32_t b2, int32_t dtype, int32_t meta,
                    const uint8_t* tile_map, hyb_layout* out, int32_t* tidx_out) {
  if (!out) return fail(HYB_ERR_INVALID_ARG, "out is NULL");
  hyb_status st = check_geometry(n, k, b1, b2, dtype, meta);
  if (st != HYB_OK) return st;
  const int64_t tn = n / b1, tk = k / b2, T = tn * tk;
  if (T > 0 && !tile_map) return fail(HYB_ERR_INVALID_ARG, "tile_map is NULL");
  if (T >= (int64_t(1) << 31)) return fail(HYB_ERR_SHAPE, "too many tiles");
  int64_t nd = 0, ns = 0;
  for (int64_t t = 0; t < T; ++t) {
    if (tile_map[t] > 1)
      return fail(HYB_ERR_INVALID_ARG, "tile_map[%lld] = %u, must be 0 or 1", (long long)t, tile_map[t]);
  }
  for (int64_t t = 0; t < T; ++t) {
    if (tile_map[t]) {
      if (tidx_out) tidx_out[t] = ~int32_t(ns);
      ++ns;
    } else {
      if (tidx_out) tidx_out[t] = int32_t(nd);
      ++nd;
    }
  }
  hyb_layout L{};
  L.magic = HYB_MAGIC;
  L.version = HYB_VERSION;
  L.n = n;
  L.k = k;
  L.b1 = b1;
  L.b2 = b2;
  L.dtype = dtype;
  L.meta = meta;
  L.tiles_n = tn;
  L.tiles_k = tk;
  L.n_dense = nd;
  L.n_sparse = ns;
  fill_sizes(&L);
  *out = L;
  return ok();
}

hyb_status hyb_layout_check(const hyb_layout* layout) {
  const hyb_status st = check_layout(layout, false);
  return st == HYB_OK ? ok() : st;
}

hyb_status hyb_pack(const hyb_layout* layout, const void* w, int64_t ldw, const hyb_packed* dst,
                    void* stream) {
  hyb_status st = check_layout(layout, true);
  if (st != HYB_OK) return st;
  if (ldw < 0) return fail(HYB_ERR_INVALID_ARG, "w row stride %lld is negative", (long long)ldw);
  if (layout->n == 0 || layout->k == 0) return ok();
  st = check_packed(layout, dst);
  if (st != HYB_OK) return st;
  st = check_matrix_arg(w, layout->n, layout->k, ldw, "w");
  if (st != HYB_OK) return st;
  return hip_status(hyb::launch_pack(*layout, w, ldw, *dst, static_cast<hipStream_t>(stream)),
                    "pack launch");
}

hyb_status hyb_unpack(const hyb_layout* layout, const hyb_packed* src, void* w_out, int64_t ldw,
                      void* stream) {
  hyb_status st = check_layout(layout, true);
  if (st != HYB_OK) return st;
  if (ldw < 0) return fail(HYB_ERR_INVALID_ARG, "w_out row stride %lld is negative", (long long)ldw);
  if (layout->n == 0 || layout->k == 0) return ok();
  st = check_packed(layout, src);
  if (st != HYB_OK) return st;
  st = check_matrix_arg(w_out, layout->n, layout->k, ldw, "w_out");
  if (st != HYB_OK) return st;
  return hip_status(hyb::launch_unpack(*layout, *src, w_out, ldw, static_cast<hipStream_t>(stream)),
                    "unpack launch");
}

namespace {

// The decode kernel itself (k_gemv), 0 <= m <= 16.
hyb_status gemv_decode(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m, int64_t ldx,
                       void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, hyb::kMaxGemvM);
  if (st != HYB_OK) return st;
  if (m == 0 || layout->n == 0) return ok();
  if (int64_t(m) * ldx * 2 >= (int64_t(1) << 31))
    return fail(HYB_ERR_UNSUPPORTED, "decode kernel needs m * ldx * 2 < 2^31 bytes of x");
  return hip_status(hyb::launch_gemv(*layout, *w, x, m, ldx, y, y_dtype, ldy,
                                     static_cast<hipStream_t>(stream)),
                    "gemv launch");
}

// Whether m tokens on this matrix run the decode kernel (the crossover of
// hyb_gemm; a NULL or invalid layout takes the decode path, whose checks
// report it).
bool decode_route(const hyb_layout* layout, int32_t m) {
  return m <= hyb::kGemvCrossoverM || !layout || check_layout(layout, true) != HYB_OK ||
         (m <= hyb::kMaxGemvM && hyb::gemv_preferred(*layout, m));
}

}  // namespace

hyb_status hyb_gemv(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                    int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  // 9-16 tokens where the decode kernel is VALU-bound run on the matrix
  // cores, as in hyb_gemm (the 16-token decode kernel: 35 us on 14336 x
  // 4096 against 19 us for the register-fed matrix-core kernel).
  if (m > hyb::kMaxGemvM || decode_route(layout, m)) return gemv_decode(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  return hyb_gemm_mfma(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
}

hyb_status hyb_gemv_grouped(int32_t count, const hyb_layout* layouts, const hyb_packed* w, const void* x,
                            int32_t m, int64_t ldx, void* const* y, int32_t y_dtype, const int64_t* ldy,
                            void* stream) {
  if (count < 0 || count > hyb::kMaxGroup)
    return fail(HYB_ERR_SHAPE, "count = %d outside [0, %d]", count, hyb::kMaxGroup);
  if (count == 0) return ok();
  if (!layouts || !w || !y || !ldy) return fail(HYB_ERR_INVALID_ARG, "layouts, w, y or ldy is NULL");
  int64_t slabs = 0;
  for (int32_t g = 0; g < count; ++g) {
    hyb_status st = check_product(&layouts[g], &w[g], x, m, ldx, y[g], y_dtype, ldy[g], hyb::kMaxGemvM);
    if (st != HYB_OK) {
      const std::string detail = g_last_error;
      return fail(st, "matrix %d: %s", g, detail.c_str());
    }
    const hyb_layout& L = layouts[g];
    const hyb_layout& L0 = layouts[0];
    if (L.k != L0.k || L.b2 != L0.b2 || L.dtype != L0.dtype || L.meta != L0.meta)
      return fail(HYB_ERR_INVALID_ARG, "matrix %d differs from matrix 0 in k, b2, dtype or metadata kind", g);
    slabs += L.n / 16;
  }
  if (m == 0 || slabs == 0) return ok();
  if (slabs >= (int64_t(1) << 31)) return fail(HYB_ERR_UNSUPPORTED, "too many rows for one launch");
  if (int64_t(m) * ldx * 2 >= (int64_t(1) << 31))
    return fail(HYB_ERR_UNSUPPORTED, "decode kernel needs m * ldx * 2 < 2^31 bytes of x");
  // Matrices that hyb_gemv would run on the matrix cores (9-16 tokens on
  // long matrices) take that kernel, one launch each, so every result stays
  // bitwise that of hyb_gemv; the rest share the grouped decode launch.  The
  // matrix-core limits are checked for all of them before anything is
  // enqueued.
  for (int32_t g = 0; g < count; ++g) {
    if (layouts[g].n == 0 || decode_route(&layouts[g], m)) continue;
    const hyb_status st = check_mfma_limits(m, ldx);
    if (st != HYB_OK) return st;
  }
  hyb_layout dl[hyb::kMaxGroup];
  hyb_packed dp[hyb::kMaxGroup];
  void* dy[hyb::kMaxGroup];
  int64_t dldy[hyb::kMaxGroup];
  int32_t nd = 0;
  for (int32_t g = 0; g < count; ++g) {
    if (layouts[g].n == 0) continue;
    if (decode_route(&layouts[g], m)) {
      dl[nd] = layouts[g];
      dp[nd] = w[g];
      dy[nd] = y[g];
      dldy[nd] = ldy[g];
      ++nd;
    } else {
      const hyb_status st = hyb_gemm_mfma(&layouts[g], &w[g], x, m, ldx, y[g], y_dtype, ldy[g], stream);
      if (st != HYB_OK) return st;
    }
  }
  if (nd == 0) return ok();
  return hip_status(hyb::launch_gemv_grouped(nd, dl, dp, x, m, ldx, dy, y_dtype, dldy,
                                             static_cast<hipStream_t>(stream)),
                    "grouped gemv launch");
}

hyb_status hyb_lowrank_project(const void* v, int64_t ldv, int32_t rank, int64_t k, int32_t dtype,
                               const void* x, int32_t m, int64_t ldx, float* t, int64_t ldt, void* stream) {
  if (dtype != HYB_BF16 && dtype != HYB_F16) return fail(HYB_ERR_DTYPE, "dtype %d must be bf16 or f16", dtype);
  if (rank < 0 || rank > hyb::kMaxRank) return fail(HYB_ERR_SHAPE, "rank = %d must be in [0, %d]", rank, hyb::kMaxRank);
  if (k < 0 || k % 8 != 0) return fail(HYB_ERR_SHAPE, "k = %lld must be a non-negative multiple of 8", (long long)k);
  if (m < 0 || m > 16 * 65535) return fail(HYB_ERR_SHAPE, "m = %d must be in [0, %d]", m, 16 * 65535);
  if (rank == 0 || m == 0) return ok();
  if (!t || !aligned(t, 4)) return fail(HYB_ERR_INVALID_ARG, "t is NULL or misaligned");
  if (ldt < rank) return fail(HYB_ERR_INVALID_ARG, "t row stride %lld must be >= rank", (long long)ldt);
  if (k > 0) {
    if (!v || !aligned(v, 16)) return fail(HYB_ERR_INVALID_ARG, "v is NULL or not 16-byte aligned");
    if (ldv < k || ldv % 8 != 0)
      return fail(HYB_ERR_INVALID_ARG, "v row stride %lld must be >= k and a multiple of 8", (long long)ldv);
    if (!x || !aligned(x, 16)) return fail(HYB_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
    if (ldx < k || ldx % 8 != 0)
      return fail(HYB_ERR_INVALID_ARG, "x row stride %lld must be >= k and a multiple of 8", (long long)ldx);
  }
  return hip_status(hyb::launch_lr_project(v, ldv, rank, k, dtype, x, m, ldx, t, ldt,
                                           static_cast<hipStream_t>(stream)),
                    "low-rank projection launch");
}

namespace {

// Checks of the low-rank operands shared by the decode and prefill entry
// points (rank > 0, m > 0).
hyb_status check_lowrank(const float* t, int64_t ldt, const void* u, int64_t ldu, int32_t rank) {
  if (!t || !aligned(t, 16)) return fail(HYB_ERR_INVALID_ARG, "t is NULL or not 16-byte aligned");
  if (ldt < rank || ldt % 4 != 0)
    return fail(HYB_ERR_INVALID_ARG, "t row stride %lld must be >= rank and a multiple of 4", (long long)ldt);
  if (!u || !aligned(u, 16)) return fail(HYB_ERR_INVALID_ARG, "u is NULL or not 16-byte aligned");
  if (ldu < rank || ldu % 8 != 0)
    return fail(HYB_ERR_INVALID_ARG, "u row stride %lld must be >= rank and a multiple of 8", (long long)ldu);
  return HYB_OK;
}

hyb_status check_rank(int32_t rank) {
  if (rank < 0 || rank > hyb::kMaxRank || rank % 8 != 0)
    return fail(HYB_ERR_SHAPE, "rank = %d must be a multiple of 8 in [0, %d]", rank, hyb::kMaxRank);
  return HYB_OK;
}

}  // namespace

namespace {

// The fused decode kernel (k_gemv with the low-rank epilogue), 0 <= m <= 16.
hyb_status gemv_lowrank_decode(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                               int64_t ldx, const float* t, int64_t ldt, const void* u, int64_t ldu, int32_t rank,
                               void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, hyb::kMaxGemvM);
  if (st != HYB_OK) return st;
  if ((st = check_rank(rank)) != HYB_OK) return st;
  if (rank == 0) return gemv_decode(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  if (m == 0 || layout->n == 0) return ok();
  if ((st = check_lowrank(t, ldt, u, ldu, rank)) != HYB_OK) return st;
  if (int64_t(m) * ldx * 2 >= (int64_t(1) << 31))
    return fail(HYB_ERR_UNSUPPORTED, "decode kernel needs m * ldx * 2 < 2^31 bytes of x");
  return hip_status(hyb::launch_gemv_lowrank(*layout, *w, x, m, ldx, t, ldt, u, ldu, rank, y, y_dtype, ldy,
                                             static_cast<hipStream_t>(stream)),
                    "low-rank gemv launch");
}

}  // namespace

hyb_status hyb_gemv_lowrank(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                            int64_t ldx, const float* t, int64_t ldt, const void* u, int64_t ldu, int32_t rank,
                            void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (m > hyb::kMaxGemvM || decode_route(layout, m))
    return gemv_lowrank_decode(layout, w, x, m, ldx, t, ldt, u, ldu, rank, y, y_dtype, ldy, stream);
  return hyb_gemm_lowrank(layout, w, x, m, ldx, t, ldt, u, ldu, rank, y, y_dtype, ldy, stream);
}


hyb_status hyb_gemm_lowrank(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                            int64_t ldx, const float* t, int64_t ldt, const void* u, int64_t ldu, int32_t rank,
                            void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (m >= 0 && m <= hyb::kMaxGemvM && decode_route(layout, m))
    return gemv_lowrank_decode(layout, w, x, m, ldx, t, ldt, u, ldu, rank, y, y_dtype, ldy, stream);
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, INT32_MAX);
  if (st != HYB_OK) return st;
  if ((st = check_rank(rank)) != HYB_OK) return st;
  if (rank == 0) return hyb_gemm(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  if (layout->n == 0) return ok();
  if ((st = check_lowrank(t, ldt, u, ldu, rank)) != HYB_OK) return st;
  if ((st = check_mfma_limits(m, ldx)) != HYB_OK) return st;
  const std::pair<void*, size_t> ws = stream_workspace(*layout, m, stream);
  return hip_status(hyb::launch_gemm(*layout, *w, x, m, ldx, y, y_dtype, ldy, static_cast<hipStream_t>(stream),
                                     ws.first, ws.second, t, ldt, u, ldu, rank),
                    "low-rank gemm launch");
}

hyb_status hyb_gemm_lowrank_ws(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                               int64_t ldx, const float* t, int64_t ldt, const void* u, int64_t ldu, int32_t rank,
                               void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (m >= 0 && m <= hyb::kMaxGemvM && decode_route(layout, m))
    return gemv_lowrank_decode(layout, w, x, m, ldx, t, ldt, u, ldu, rank, y, y_dtype, ldy, stream);
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, INT32_MAX);
  if (st != HYB_OK) return st;
  if ((st = check_rank(rank)) != HYB_OK) return st;
  if (workspace_bytes > 0 && (!workspace || !aligned(workspace, 16)))
    return fail(HYB_ERR_INVALID_ARG, "workspace is NULL or not 16-byte aligned with workspace_bytes = %zu",
                workspace_bytes);
  if (rank == 0)
    return hyb_gemm_ws(layout, w, x, m, ldx, y, y_dtype, ldy, workspace, workspace_bytes, stream);
  if (layout->n == 0) return ok();
  if ((st = check_lowrank(t, ldt, u, ldu, rank)) != HYB_OK) return st;
  if ((st = check_mfma_limits(m, ldx)) != HYB_OK) return st;
  const size_t need = hyb::split_workspace_bytes(hyb::gemm_route(*layout, m, hyb::device_cus()));
  if (workspace_bytes > 0 && workspace_bytes < need)
    return fail(HYB_ERR_INVALID_ARG, "workspace_bytes = %zu, this product needs %zu (or 0: unsplit)",
                workspace_bytes, need);
  return hip_status(hyb::launch_gemm(*layout, *w, x, m, ldx, y, y_dtype, ldy, static_cast<hipStream_t>(stream),
                                     workspace_bytes > 0 ? workspace : nullptr, workspace_bytes, t, ldt, u, ldu,
                                     rank),
                    "low-rank gemm launch");
}

hyb_status hyb_gemm_mfma(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                         int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, INT32_MAX);
  if (st != HYB_OK) return st;
  if (m == 0 || layout->n == 0) return ok();
  if ((st = check_mfma_limits(m, ldx)) != HYB_OK) return st;
  const std::pair<void*, size_t> ws = stream_workspace(*layout, m, stream);
  return hip_status(hyb::launch_gemm(*layout, *w, x, m, ldx, y, y_dtype, ldy, static_cast<hipStream_t>(stream),
                                     ws.first, ws.second),
                    "gemm launch");
}

hyb_status hyb_gemm(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m,
                    int64_t ldx, void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (m >= 0 && m <= hyb::kMaxGemvM && decode_route(layout, m))
    return gemv_decode(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  return hyb_gemm_mfma(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
}

hyb_status hyb_gemm_noalloc(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m, int64_t ldx,
                            void* y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (m >= 0 && m <= hyb::kMaxGemvM && decode_route(layout, m))
    return gemv_decode(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, INT32_MAX);
  if (st != HYB_OK) return st;
  if (m == 0 || layout->n == 0) return ok();
  if ((st = check_mfma_limits(m, ldx)) != HYB_OK) return st;
  const size_t need = hyb::split_workspace_bytes(hyb::gemm_route(*layout, m, hyb::device_cus()));
  if (need > hyb::kSplitMaxBytes)
    return fail(HYB_ERR_UNSUPPORTED, "this product needs %zu bytes of scratch, above the %zu bytes held per device",
                need, hyb::kSplitMaxBytes);
  void* ws = nullptr;
  if (need > 0) {
    if ((st = hip_status(hyb::split_scratch(&ws), "device scratch address")) != HYB_OK) return st;
  }
  return hip_status(hyb::launch_gemm(*layout, *w, x, m, ldx, y, y_dtype, ldy, static_cast<hipStream_t>(stream),
                                     ws, need > 0 ? hyb::kSplitMaxBytes : 0),
                    "gemm launch");
}

hyb_status hyb_gemm_workspace_size(const hyb_layout* layout, int32_t m, size_t* bytes) {
  hyb_status st = check_layout(layout, true);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARG, "bytes is NULL");
  if (m < 0) return fail(HYB_ERR_SHAPE, "m = %d is negative", m);
  *bytes = 0;
  if (m == 0 || layout->n == 0) return ok();
  const hyb::GemmRoute r = hyb::gemm_route_device(*layout, m);
  *bytes = hyb::split_workspace_bytes(r);
  return ok();
}

hyb_status hyb_gemm_ws(const hyb_layout* layout, const hyb_packed* w, const void* x, int32_t m, int64_t ldx,
                       void* y, int32_t y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (m >= 0 && m <= hyb::kMaxGemvM && decode_route(layout, m))
    return gemv_decode(layout, w, x, m, ldx, y, y_dtype, ldy, stream);
  hyb_status st = check_product(layout, w, x, m, ldx, y, y_dtype, ldy, INT32_MAX);
  if (st != HYB_OK) return st;
  if (workspace_bytes > 0 && (!workspace || !aligned(workspace, 16)))
    return fail(HYB_ERR_INVALID_ARG, "workspace is NULL or not 16-byte aligned with workspace_bytes = %zu",
                workspace_bytes);
  if (m == 0 || layout->n == 0) return ok();
  if ((st = check_mfma_limits(m, ldx)) != HYB_OK) return st;
  const size_t need = hyb::split_workspace_bytes(hyb::gemm_route(*layout, m, hyb::device_cus()));
  if (workspace_bytes > 0 && workspace_bytes < need)
    return fail(HYB_ERR_INVALID_ARG, "workspace_bytes = %zu, this product needs %zu (or 0: unsplit)",
                workspace_bytes, need);
  return hip_status(hyb::launch_gemm(*layout, *w, x, m, ldx, y, y_dtype, ldy, static_cast<hipStream_t>(stream),
                                     workspace_bytes > 0 ? workspace : nullptr, workspace_bytes),
                    "gemm launch");
}

hyb_status hyb_gemm_shape(const hyb_layout* layout, int32_t m, int32_t* out) {
  hyb_status st = check_layout(layout, true);
  if (st != HYB_OK) return st;
  if (!out) return fail(HYB_ERR_INVALID_ARG, "out is NULL");
  if (m < 1) return fail(HYB_ERR_SHAPE, "m = %d, the query needs m >= 1", m);
  const hyb::GemmRoute r = hyb::gemm_route_device(*layout, m);
  // hyb_gemm rejects what the matrix-core kernels cannot launch; so does
  // the query (same limit as check_mfma_limits).
  if (r.kernel != hyb::kRouteDecode && (int64_t(m) + 15) / 16 > 65535 * 8)
    return fail(HYB_ERR_UNSUPPORTED, "m = %d too large for one launch", m);
  out[0] = r.kernel;
  out[1] = r.mb;
  out[2] = r.waves;
  out[3] = r.rg;
  return ok();
}

hyb_status hyb_stream_read(const void* p, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (bytes < 0 || bytes >= (int64_t(1) << 31)) return fail(HYB_ERR_SHAPE, "bytes must be in [0, 2^31)");
  if (grid < 1 || grid > 65535) return fail(HYB_ERR_INVALID_ARG, "grid must be in [1, 65535]");
  if (!sink || !aligned(sink, 4)) return fail(HYB_ERR_INVALID_ARG, "sink is NULL or misaligned");
  if (bytes > 0 && (!p || !aligned(p, 16))) return fail(HYB_ERR_INVALID_ARG, "p is NULL or not 16-byte aligned");
  return hip_status(hyb::launch_stream_read(p, bytes, sink, grid, static_cast<hipStream_t>(stream)),
                    "stream read launch");
}

}  // extern "C"
