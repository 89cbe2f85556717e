// The C ABI (include/moe.h): argument checks on the host, then launches on the
// caller's stream. Nothing here allocates or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char *fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    g_last_error = msg;
    return st;
}

moe_status hip_fail(hipError_t e, const char *where) {
    return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOE_REQUIRE(cond, ...)                         \
    do {                                               \
        if (!(cond)) return fail(MOE_EINVAL, __VA_ARGS__); \
    } while (0)

// The kernels move rows in 16-byte vectors; NULL counts as aligned.
template <class... P>
bool aligned16(P... p) {
    return (((reinterpret_cast<uintptr_t>(p) & 15u) == 0) && ...);
}
#define MOE_REQUIRE_ALIGNED(...) MOE_REQUIRE(aligned16(__VA_ARGS__), "device buffers must be 16-byte aligned")

int64_t by_factor(const moe_shape &s) {
    // ceil(k * S * |f| / E), the capacity a factor of |f| gives
    return static_cast<int64_t>(std::ceil((static_cast<double>(s.k) * static_cast<double>(s.S) *
                                           std::fabs(s.capacity_factor)) / static_cast<double>(s.E)));
}

int64_t cap_bound(const moe_shape &s) {
    int64_t c;
    if (s.capacity_factor > 0) c = by_factor(s);
    else if (s.capacity_factor == 0) c = s.S;
    else c = std::min<int64_t>(by_factor(s), s.S);
    return c < 1 ? 1 : c;
}

int32_t num_tiles(const moe_shape &s) { return (s.S + moe::kRouteTile - 1) / moe::kRouteTile; }

// Workspace of routing and the forwards: routing's per-tile route counts; the
// Residual-MoE branch reuses 8 bytes of it after routing.
size_t forward_ws_bytes(const moe_shape &s) {
    const size_t n = static_cast<size_t>(s.E) * s.k * num_tiles(s);
    return std::max<size_t>(256, ((n * sizeof(int32_t)) + 255) & ~static_cast<size_t>(255));
}

// One workspace serves routing (per-tile route counts) and the gate backward
// (auxiliary-loss partials and dWg slice partials); they are never live together.
size_t ws_bytes_needed(const moe_shape &s) {
    return std::max(forward_ws_bytes(s), moe::gate_grad_ws_bytes(s.S, s.M, s.E));
}

moe_status check_ws_bytes(const void *ws, size_t ws_bytes, size_t need) {
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(MOE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? 0 : ws_bytes);
    return MOE_OK;
}

moe_status check_forward_ws(const moe_shape &s, const void *ws, size_t ws_bytes) {
    return check_ws_bytes(ws, ws_bytes, forward_ws_bytes(s));
}

moe_status check_ws(const moe_shape &s, const void *ws, size_t ws_bytes) {
    return check_ws_bytes(ws, ws_bytes, ws_bytes_needed(s));
}

moe_status check_shape(const moe_shape *sp) {
    if (sp == nullptr) return fail(MOE_EINVAL, "shape is NULL");
    const moe_shape &s = *sp;
    if (s.S < 0 || s.M <= 0 || s.E <= 0 || s.H <= 0 || s.k <= 0)
        return fail(MOE_EINVAL, "sizes must be positive (S >= 0): S=%d M=%d E=%d k=%d H=%d", s.S, s.M, s.E, s.k, s.H);
    if (s.k > s.E) return fail(MOE_EINVAL, "k=%d exceeds E=%d", s.k, s.E);
    if (!std::isfinite(s.capacity_factor)) return fail(MOE_EINVAL, "capacity_factor is not finite");
    if (s.dtype != MOE_DT_F32 && s.dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "unknown dtype %d", s.dtype);
    if (s.act != MOE_ACT_RELU && s.act != MOE_ACT_GELU) return fail(MOE_EINVAL, "unknown activation %d", s.act);
    if (s.k > moe::kMaxK) return fail(MOE_EUNSUPPORTED, "k=%d above the supported %d", s.k, moe::kMaxK);
    if (s.E > moe::kMaxE) return fail(MOE_EUNSUPPORTED, "E=%d above the supported %d", s.E, moe::kMaxE);
    if (s.M % 64 != 0 || s.H % 64 != 0)
        return fail(MOE_EUNSUPPORTED, "M=%d and H=%d must be multiples of 64", s.M, s.H);
    if (static_cast<int64_t>(s.S) * s.k >= (int64_t(1) << 31))
        return fail(MOE_EUNSUPPORTED, "S*k=%lld routes exceed int32 indices", (long long)s.S * s.k);
    const int64_t rows = static_cast<int64_t>(s.E) * cap_bound(s);
    if (rows >= (int64_t(1) << 31))
        return fail(MOE_EUNSUPPORTED, "E*C bound %lld rows exceeds int32 slot indices", (long long)rows);
    if (cap_bound(s) / 128 >= 65535) return fail(MOE_EUNSUPPORTED, "capacity bound too large for the GEMM grid");
    return MOE_OK;
}

hipStream_t as_stream(void *p) { return reinterpret_cast<hipStream_t>(p); }

}  // namespace

extern "C" {

moe_status moe_validate(const moe_shape *shape) { return check_shape(shape); }

moe_status moe_capacity_bound(const moe_shape *shape, int32_t *cmax_host) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(cmax_host != nullptr, "cmax_host is NULL");
    *cmax_host = static_cast<int32_t>(cap_bound(*shape));
    return MOE_OK;
}

moe_status moe_workspace_size(const moe_shape *shape, size_t *bytes_host) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(bytes_host != nullptr, "bytes_host is NULL");
    *bytes_host = ws_bytes_needed(*shape);
    return MOE_OK;
}

moe_status moe_gate_project(const moe_shape *shape, const void *x, const float *Wg, float *logits, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if (s.S > 0) MOE_REQUIRE(x && Wg && logits, "x, Wg and logits must be non-NULL");
    MOE_REQUIRE_ALIGNED(x, Wg, logits);
    if (!moe::gate_supported(s.M, s.E, s.dtype))
        return fail(MOE_EUNSUPPORTED, "gate projection tiles for M=%d, E=%d do not fit in LDS", s.M, s.E);
    hipError_t e = moe::launch_gate_project(s, x, Wg, logits, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "gate projection");
}

moe_status moe_route(const moe_shape *shape, const float *logits, int32_t *idx, int32_t *loc, float *gates,
                     int32_t *needed, int32_t *fill, int32_t *capacity, int32_t *slot_route, void *ws,
                     size_t ws_bytes, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(needed && fill && capacity, "needed, fill and capacity must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(logits && idx && loc && gates, "logits, idx, loc and gates must be non-NULL");
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(logits, idx, loc, gates, needed, fill, capacity, slot_route, ws);
    moe::RouteWs w{static_cast<int32_t *>(ws), num_tiles(s)};
    hipError_t e = moe::launch_route(s, logits, idx, loc, gates, needed, fill, capacity, slot_route, w, by_factor(s),
                                     as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "route");
}

moe_status moe_encode(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                      const int32_t *fill, const int32_t *capacity, void *buf, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(fill && capacity && buf, "fill, capacity and buf must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc, "x, idx and loc must be non-NULL");
    MOE_REQUIRE_ALIGNED(x, idx, loc, fill, capacity, buf);
    hipError_t e = moe::launch_encode(s, x, idx, loc, fill, capacity, buf, static_cast<int32_t>(cap_bound(s)),
                                      as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "encode");
}

moe_status moe_expert_ffn(const moe_shape *shape, const void *buf, const void *W1, const void *b1, const void *W2,
                          const void *b2, const int32_t *fill, const int32_t *capacity, void *pre, void *h, void *y,
                          void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(buf && W1 && W2 && fill && capacity && h && y, "buf, W1, W2, fill, capacity, h and y must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(buf, W1, b1, W2, b2, fill, capacity, pre, h, y);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    hipError_t e = moe::launch_fc1(s, buf, W1, b1, fill, capacity, pre, h, cmax, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "expert fc1");
    e = moe::launch_fc2(s, h, W2, b2, fill, capacity, y, cmax, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc2");
}

static moe_status check_nvfp4_ffn(const moe_shape &s) {
    if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "NVFP4 experts take bf16 tokens");
    return MOE_OK;
}

moe_status moe_expert_ffn_nvfp4(const moe_shape *shape, const void *buf, const void *W1_codes, const void *W1_scales,
                                const float *W1_g, const void *b1, const void *W2_codes, const void *W2_scales,
                                const float *W2_g, const void *b2, const int32_t *fill, const int32_t *capacity,
                                void *pre, void *h, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_nvfp4_ffn(s)) != MOE_OK) return st;
    MOE_REQUIRE(buf && W1_codes && W1_scales && W1_g && W2_codes && W2_scales && W2_g && fill && capacity && h && y,
                "buf, the weights' codes, scales and g, fill, capacity, h and y must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(buf, W1_codes, W1_scales, W1_g, b1, W2_codes, W2_scales, W2_g, b2, fill, capacity, pre, h, y);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    hipError_t e = moe::launch_fc1_nvfp4(s, buf, static_cast<const uint8_t *>(W1_codes),
                                         static_cast<const uint8_t *>(W1_scales), W1_g, b1, fill, capacity, pre, h,
                                         cmax, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "expert fc1 (NVFP4)");
    e = moe::launch_fc2_nvfp4(s, h, static_cast<const uint8_t *>(W2_codes), static_cast<const uint8_t *>(W2_scales),
                              W2_g, b2, fill, capacity, y, cmax, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc2 (NVFP4)");
}

moe_status moe_expert_fc1_nvfp4(const moe_shape *shape, const void *buf, const void *W1_codes, const void *W1_scales,
                                const float *W1_g, const void *b1, const int32_t *fill, const int32_t *capacity,
                                void *pre, void *h, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_nvfp4_ffn(s)) != MOE_OK) return st;
    MOE_REQUIRE(buf && W1_codes && W1_scales && W1_g && fill && capacity && h,
                "buf, W1's codes, scales and g, fill, capacity and h must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE_ALIGNED(buf, W1_codes, W1_scales, W1_g, b1, fill, capacity, pre, h);
    hipError_t e = moe::launch_fc1_nvfp4(s, buf, static_cast<const uint8_t *>(W1_codes),
                                         static_cast<const uint8_t *>(W1_scales), W1_g, b1, fill, capacity, pre, h,
                                         static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc1 (NVFP4)");
}

moe_status moe_expert_fc2_nvfp4(const moe_shape *shape, const void *h, const void *W2_codes, const void *W2_scales,
                                const float *W2_g, const void *b2, const int32_t *fill, const int32_t *capacity,
                                void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_nvfp4_ffn(s)) != MOE_OK) return st;
    MOE_REQUIRE(h && W2_codes && W2_scales && W2_g && fill && capacity && y,
                "h, W2's codes, scales and g, fill, capacity and y must be non-NULL");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(h, W2_codes, W2_scales, W2_g, b2, fill, capacity, y);
    hipError_t e = moe::launch_fc2_nvfp4(s, h, static_cast<const uint8_t *>(W2_codes),
                                         static_cast<const uint8_t *>(W2_scales), W2_g, b2, fill, capacity, y,
                                         static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc2 (NVFP4)");
}

moe_status moe_expert_ffn_window(const moe_shape *shape, const void *buf, const void *W1, const void *b1,
                                 const void *W2, const void *b2, const int32_t *fill, const int32_t *capacity,
                                 int32_t slot_begin, int32_t slot_end, void *pre, void *h, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "the slot-window FFN takes bf16 data");
    MOE_REQUIRE(slot_begin >= 0 && slot_end >= slot_begin, "bad slot window [%d, %d)", slot_begin, slot_end);
    MOE_REQUIRE(buf && W1 && W2 && fill && capacity && h && y, "buf, W1, W2, fill, capacity, h and y must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(buf, W1, b1, W2, b2, fill, capacity, pre, h, y);
    if (slot_end == slot_begin) return MOE_OK;
    hipError_t e = moe::launch_ffn_window(s, buf, W1, b1, W2, b2, fill, capacity, pre, h, y,
                                          static_cast<int32_t>(cap_bound(s)), slot_begin, slot_end, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert ffn window");
}

moe_status moe_expert_fc1(const moe_shape *shape, const void *buf, const void *W1, const void *b1,
                          const int32_t *fill, const int32_t *capacity, void *pre, void *h, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(buf && W1 && fill && capacity && h, "buf, W1, fill, capacity and h must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE_ALIGNED(buf, W1, b1, fill, capacity, pre, h);
    hipError_t e = moe::launch_fc1(s, buf, W1, b1, fill, capacity, pre, h, static_cast<int32_t>(cap_bound(s)),
                                   as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc1");
}

moe_status moe_expert_fc2(const moe_shape *shape, const void *h, const void *W2, const void *b2,
                          const int32_t *fill, const int32_t *capacity, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(h && W2 && fill && capacity && y, "h, W2, fill, capacity and y must be non-NULL");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(h, W2, b2, fill, capacity, y);
    hipError_t e = moe::launch_fc2(s, h, W2, b2, fill, capacity, y, static_cast<int32_t>(cap_bound(s)),
                                   as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "expert fc2");
}

moe_status moe_decode(const moe_shape *shape, const void *y, const float *gates, const int32_t *idx,
                      const int32_t *loc, const int32_t *capacity, void *out, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(capacity != nullptr, "capacity is NULL");
    if (s.S > 0) MOE_REQUIRE(y && gates && idx && loc && out, "y, gates, idx, loc and out must be non-NULL");
    MOE_REQUIRE_ALIGNED(y, gates, idx, loc, capacity, out);
    hipError_t e = moe::launch_decode(s, y, gates, idx, loc, capacity, out, false, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "decode");
}

moe_status moe_mx_quantize(int32_t fmt, int64_t rows, int32_t K, int32_t dtype, const void *src, void *codes,
                           void *scales, void *stream) {
    MOE_REQUIRE(fmt == MOE_MX_FP8 || fmt == MOE_MX_FP4, "unknown MX format %d", fmt);
    MOE_REQUIRE(dtype == MOE_DT_F32 || dtype == MOE_DT_BF16, "unknown dtype %d", dtype);
    MOE_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, "rows must be >= 0 and K a positive multiple of 32");
    MOE_REQUIRE(rows * (K / 32) < (int64_t(1) << 40), "matrix too large");
    if (rows > 0) MOE_REQUIRE(src && codes && scales, "src, codes and scales must be non-NULL");
    MOE_REQUIRE_ALIGNED(src, codes, scales);
    hipError_t e = moe::launch_mx_quantize(fmt, rows, K, dtype, src, static_cast<uint8_t *>(codes),
                                           static_cast<uint8_t *>(scales), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "MX quantisation");
}

}  // extern "C"

namespace {

moe_status check_mx_shape(const moe_shape &s, int wfmt) {
    if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "MX experts take bf16 tokens and outputs");
    if (wfmt != MOE_MX_FP8 && wfmt != MOE_MX_FP4) return fail(MOE_EINVAL, "unknown MX weight format %d", wfmt);
    if (s.M % 128 != 0 || s.H % 128 != 0)
        return fail(MOE_EUNSUPPORTED, "MX experts need M and H multiples of 128 (M=%d, H=%d)", s.M, s.H);
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_encode_mx(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                         const int32_t *fill, const int32_t *capacity, void *buf_codes, void *buf_scales,
                         void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_mx_shape(s, MOE_MX_FP8)) != MOE_OK) return st;
    MOE_REQUIRE(fill && capacity && buf_codes && buf_scales, "fill, capacity, buf_codes and buf_scales must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc, "x, idx and loc must be non-NULL");
    MOE_REQUIRE_ALIGNED(x, idx, loc, fill, capacity, buf_codes, buf_scales);
    hipError_t e = moe::launch_encode_mx(s, x, idx, loc, fill, capacity, static_cast<uint8_t *>(buf_codes),
                                         static_cast<uint8_t *>(buf_scales), static_cast<int32_t>(cap_bound(s)),
                                         as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "MX encode");
}

moe_status moe_expert_ffn_mx(const moe_shape *shape, int32_t wfmt, const void *buf_codes, const void *buf_scales,
                             const void *W1_codes, const void *W1_scales, const void *b1, const void *W2_codes,
                             const void *W2_scales, const void *b2, const int32_t *fill, const int32_t *capacity,
                             void *h_codes, void *h_scales, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_mx_shape(s, wfmt)) != MOE_OK) return st;
    MOE_REQUIRE(buf_codes && buf_scales && W1_codes && W1_scales && W2_codes && W2_scales && fill && capacity &&
                    h_codes && h_scales && y,
                "buffers, weights, fill, capacity, h and y must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(buf_codes, buf_scales, W1_codes, W1_scales, b1, W2_codes, W2_scales, b2, fill, capacity,
                        h_codes, h_scales, y);
    hipError_t e = moe::launch_expert_ffn_mx(
        s, wfmt, static_cast<const uint8_t *>(buf_codes), static_cast<const uint8_t *>(buf_scales),
        static_cast<const uint8_t *>(W1_codes), static_cast<const uint8_t *>(W1_scales), b1,
        static_cast<const uint8_t *>(W2_codes), static_cast<const uint8_t *>(W2_scales), b2, fill, capacity,
        static_cast<uint8_t *>(h_codes), static_cast<uint8_t *>(h_scales), y, static_cast<int32_t>(cap_bound(s)),
        as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "MX expert ffn");
}

moe_status moe_expert_fc1_mx(const moe_shape *shape, int32_t wfmt, const void *buf_codes, const void *buf_scales,
                             const void *W1_codes, const void *W1_scales, const void *b1, const int32_t *fill,
                             const int32_t *capacity, void *h_codes, void *h_scales, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_mx_shape(s, wfmt)) != MOE_OK) return st;
    MOE_REQUIRE(buf_codes && buf_scales && W1_codes && W1_scales && fill && capacity && h_codes && h_scales,
                "buffers, weights, fill, capacity and h must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE_ALIGNED(buf_codes, buf_scales, W1_codes, W1_scales, b1, fill, capacity, h_codes, h_scales);
    hipError_t e = moe::launch_fc1_mx(s, wfmt, static_cast<const uint8_t *>(buf_codes),
                                      static_cast<const uint8_t *>(buf_scales), static_cast<const uint8_t *>(W1_codes),
                                      static_cast<const uint8_t *>(W1_scales), b1, fill, capacity,
                                      static_cast<uint8_t *>(h_codes), static_cast<uint8_t *>(h_scales),
                                      static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "MX expert fc1");
}

moe_status moe_expert_fc2_mx(const moe_shape *shape, int32_t wfmt, const void *h_codes, const void *h_scales,
                             const void *W2_codes, const void *W2_scales, const void *b2, const int32_t *fill,
                             const int32_t *capacity, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_mx_shape(s, wfmt)) != MOE_OK) return st;
    MOE_REQUIRE(h_codes && h_scales && W2_codes && W2_scales && fill && capacity && y,
                "h, weights, fill, capacity and y must be non-NULL");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(h_codes, h_scales, W2_codes, W2_scales, b2, fill, capacity, y);
    hipError_t e = moe::launch_fc2_mx(s, wfmt, static_cast<const uint8_t *>(h_codes),
                                      static_cast<const uint8_t *>(h_scales), static_cast<const uint8_t *>(W2_codes),
                                      static_cast<const uint8_t *>(W2_scales), b2, fill, capacity, y,
                                      static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "MX expert fc2");
}

}  // extern "C"

namespace {

moe_status check_blk_shape(const moe_shape &s) {
    if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "block-FP8 experts take bf16 tokens and outputs");
    if (s.M % 128 != 0 || s.H % 128 != 0)
        return fail(MOE_EUNSUPPORTED, "block-FP8 experts need M and H multiples of 128 (M=%d, H=%d)", s.M, s.H);
    return MOE_OK;
}

// The forward with low-precision experts: wfmt is an MX weight format (tokens and h
// MXFP8) or kBlkFp8 (block-wise FP8 throughout); the shape was checked for it.
moe_status layer_forward_lp_impl(const moe_shape &s, int wfmt, const void *x, const float *logits_in,
                                 const float *Wg, float *logits_out, const void *W1_codes, const void *W1_scales,
                                 const void *b1, const void *W2_codes, const void *W2_scales, const void *b2,
                                 int32_t *idx, int32_t *loc, float *gates, int32_t *needed, int32_t *fill,
                                 int32_t *capacity, int32_t *slot_route, void *buf_codes, void *buf_scales,
                                 void *h_codes, void *h_scales, void *y, void *out, void *ws, size_t ws_bytes,
                                 void *stream) {
    moe_status st;
    MOE_REQUIRE(!(logits_in != nullptr && Wg != nullptr), "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(s.S == 0 || logits_in != nullptr || Wg != nullptr, "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(Wg == nullptr || logits_out != nullptr || s.S == 0, "logits_out is required with Wg");
    MOE_REQUIRE(needed && fill && capacity && buf_codes && buf_scales && W1_codes && W1_scales && W2_codes &&
                    W2_scales && h_codes && h_scales && y,
                "needed, fill, capacity, buffers and weights must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc && gates && out, "x, idx, loc, gates and out must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(x, logits_in, Wg, logits_out, W1_codes, W1_scales, b1, W2_codes, W2_scales, b2, idx, loc,
                        gates, needed, fill, capacity, slot_route, buf_codes, buf_scales, h_codes, h_scales, y, out,
                        ws);
    if (Wg != nullptr && !moe::gate_supported(s.M, s.E, s.dtype))
        return fail(MOE_EUNSUPPORTED, "gate projection tiles for M=%d, E=%d do not fit in LDS", s.M, s.E);
    hipStream_t strm = as_stream(stream);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    const float *logits = logits_in;
    hipError_t e;
    if (Wg != nullptr && s.S > 0) {
        if ((e = moe::launch_gate_project(s, x, Wg, logits_out, strm)) != hipSuccess) return hip_fail(e, "gate projection");
        logits = logits_out;
    }
    moe::RouteWs w{static_cast<int32_t *>(ws), num_tiles(s)};
    if ((e = moe::launch_route(s, logits, idx, loc, gates, needed, fill, capacity, slot_route, w, by_factor(s), strm)) !=
        hipSuccess)
        return hip_fail(e, "route");
    auto *bc = static_cast<uint8_t *>(buf_codes);
    auto *bs = static_cast<uint8_t *>(buf_scales);
    e = wfmt == moe::kBlkFp8
            ? moe::launch_encode_blk(s, x, idx, loc, fill, capacity, bc, static_cast<float *>(buf_scales), cmax, strm)
            : moe::launch_encode_mx(s, x, idx, loc, fill, capacity, bc, bs, cmax, strm);
    if (e != hipSuccess) return hip_fail(e, "low-precision encode");
    if ((e = moe::launch_expert_ffn_mx(s, wfmt, bc, bs, static_cast<const uint8_t *>(W1_codes),
                                       static_cast<const uint8_t *>(W1_scales), b1,
                                       static_cast<const uint8_t *>(W2_codes), static_cast<const uint8_t *>(W2_scales),
                                       b2, fill, capacity, static_cast<uint8_t *>(h_codes),
                                       static_cast<uint8_t *>(h_scales), y, cmax, strm)) != hipSuccess)
        return hip_fail(e, "low-precision expert ffn");
    if ((e = moe::launch_decode(s, y, gates, idx, loc, capacity, out, false, strm)) != hipSuccess)
        return hip_fail(e, "decode");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_mx(const moe_shape *shape, int32_t wfmt, const void *x, const float *logits_in,
                                const float *Wg, float *logits_out, const void *W1_codes, const void *W1_scales,
                                const void *b1, const void *W2_codes, const void *W2_scales, const void *b2,
                                int32_t *idx, int32_t *loc, float *gates, int32_t *needed, int32_t *fill,
                                int32_t *capacity, int32_t *slot_route, void *buf_codes, void *buf_scales,
                                void *h_codes, void *h_scales, void *y, void *out, void *ws, size_t ws_bytes,
                                void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if ((st = check_mx_shape(*shape, wfmt)) != MOE_OK) return st;
    return layer_forward_lp_impl(*shape, wfmt, x, logits_in, Wg, logits_out, W1_codes, W1_scales, b1, W2_codes,
                                 W2_scales, b2, idx, loc, gates, needed, fill, capacity, slot_route, buf_codes,
                                 buf_scales, h_codes, h_scales, y, out, ws, ws_bytes, stream);
}

moe_status moe_layer_forward_blockfp8(const moe_shape *shape, const void *x, const float *logits_in,
                                      const float *Wg, float *logits_out, const void *W1_codes,
                                      const float *W1_scales, const void *b1, const void *W2_codes,
                                      const float *W2_scales, const void *b2, int32_t *idx, int32_t *loc,
                                      float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                                      int32_t *slot_route, void *buf_codes, float *buf_scales, void *h_codes,
                                      float *h_scales, void *y, void *out, void *ws, size_t ws_bytes, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if ((st = check_blk_shape(*shape)) != MOE_OK) return st;
    return layer_forward_lp_impl(*shape, moe::kBlkFp8, x, logits_in, Wg, logits_out, W1_codes, W1_scales, b1,
                                 W2_codes, W2_scales, b2, idx, loc, gates, needed, fill, capacity, slot_route,
                                 buf_codes, buf_scales, h_codes, h_scales, y, out, ws, ws_bytes, stream);
}

moe_status moe_blockfp8_quantize(int64_t rows, int32_t K, int32_t brows, int32_t dtype, const void *src, void *codes,
                                 float *scales, void *stream) {
    MOE_REQUIRE(brows == 1 || brows == 128, "brows must be 1 or 128, not %d", brows);
    MOE_REQUIRE(dtype == MOE_DT_F32 || dtype == MOE_DT_BF16, "unknown dtype %d", dtype);
    MOE_REQUIRE(rows >= 0 && K > 0 && K % 128 == 0, "rows must be >= 0 and K a positive multiple of 128");
    MOE_REQUIRE(rows % brows == 0, "rows=%lld must be a multiple of brows=%d", (long long)rows, brows);
    MOE_REQUIRE(rows * (K / 128) < (int64_t(1) << 40), "matrix too large");
    if (rows > 0) MOE_REQUIRE(src && codes && scales, "src, codes and scales must be non-NULL");
    MOE_REQUIRE_ALIGNED(src, codes, scales);
    hipError_t e = moe::launch_blk_quantize(brows, rows, K, dtype, src, static_cast<uint8_t *>(codes), scales,
                                            as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "block-FP8 quantisation");
}

moe_status moe_nvfp4_quantize(int64_t rows, int32_t K, int32_t ntensor, int32_t dtype, const void *src, void *codes,
                              void *scales, float *g, void *stream) {
    MOE_REQUIRE(dtype == MOE_DT_F32 || dtype == MOE_DT_BF16, "unknown dtype %d", dtype);
    MOE_REQUIRE(rows >= 0 && K > 0 && K % 16 == 0, "rows must be >= 0 and K a positive multiple of 16");
    MOE_REQUIRE(ntensor >= 1 && ntensor <= 65535 && rows % ntensor == 0,
                "ntensor must be in [1, 65535] and divide rows=%lld", (long long)rows);
    MOE_REQUIRE(rows * (K / 16) < (int64_t(1) << 40), "matrix too large");
    if (rows > 0) MOE_REQUIRE(src && codes && scales && g, "src, codes, scales and g must be non-NULL");
    MOE_REQUIRE_ALIGNED(src, codes, scales, g);
    hipError_t e = moe::launch_nvfp4_quantize(rows, K, ntensor, dtype, src, static_cast<uint8_t *>(codes),
                                              static_cast<uint8_t *>(scales), g, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "NVFP4 quantisation");
}

moe_status moe_encode_blockfp8(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                               const int32_t *fill, const int32_t *capacity, void *buf_codes, float *buf_scales,
                               void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_blk_shape(s)) != MOE_OK) return st;
    MOE_REQUIRE(fill && capacity && buf_codes && buf_scales, "fill, capacity, buf_codes and buf_scales must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc, "x, idx and loc must be non-NULL");
    MOE_REQUIRE_ALIGNED(x, idx, loc, fill, capacity, buf_codes, buf_scales);
    hipError_t e = moe::launch_encode_blk(s, x, idx, loc, fill, capacity, static_cast<uint8_t *>(buf_codes),
                                          buf_scales, static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "block-FP8 encode");
}

moe_status moe_expert_ffn_blockfp8(const moe_shape *shape, const void *buf_codes, const float *buf_scales,
                                   const void *W1_codes, const float *W1_scales, const void *b1, const void *W2_codes,
                                   const float *W2_scales, const void *b2, const int32_t *fill,
                                   const int32_t *capacity, void *h_codes, float *h_scales, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_blk_shape(s)) != MOE_OK) return st;
    MOE_REQUIRE(buf_codes && buf_scales && W1_codes && W1_scales && W2_codes && W2_scales && fill && capacity &&
                    h_codes && h_scales && y,
                "buffers, weights, fill, capacity, h and y must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(buf_codes, buf_scales, W1_codes, W1_scales, b1, W2_codes, W2_scales, b2, fill, capacity,
                        h_codes, h_scales, y);
    hipError_t e = moe::launch_expert_ffn_mx(
        s, moe::kBlkFp8, static_cast<const uint8_t *>(buf_codes), reinterpret_cast<const uint8_t *>(buf_scales),
        static_cast<const uint8_t *>(W1_codes), reinterpret_cast<const uint8_t *>(W1_scales), b1,
        static_cast<const uint8_t *>(W2_codes), reinterpret_cast<const uint8_t *>(W2_scales), b2, fill, capacity,
        static_cast<uint8_t *>(h_codes), reinterpret_cast<uint8_t *>(h_scales), y, static_cast<int32_t>(cap_bound(s)),
        as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "block-FP8 expert ffn");
}

moe_status moe_expert_fc1_blockfp8(const moe_shape *shape, const void *buf_codes, const float *buf_scales,
                                   const void *W1_codes, const float *W1_scales, const void *b1, const int32_t *fill,
                                   const int32_t *capacity, void *h_codes, float *h_scales, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_blk_shape(s)) != MOE_OK) return st;
    MOE_REQUIRE(buf_codes && buf_scales && W1_codes && W1_scales && fill && capacity && h_codes && h_scales,
                "buffers, weights, fill, capacity and h must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE_ALIGNED(buf_codes, buf_scales, W1_codes, W1_scales, b1, fill, capacity, h_codes, h_scales);
    hipError_t e = moe::launch_fc1_mx(s, moe::kBlkFp8, static_cast<const uint8_t *>(buf_codes),
                                      reinterpret_cast<const uint8_t *>(buf_scales),
                                      static_cast<const uint8_t *>(W1_codes),
                                      reinterpret_cast<const uint8_t *>(W1_scales), b1, fill, capacity,
                                      static_cast<uint8_t *>(h_codes), reinterpret_cast<uint8_t *>(h_scales),
                                      static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "block-FP8 expert fc1");
}

moe_status moe_expert_fc2_blockfp8(const moe_shape *shape, const void *h_codes, const float *h_scales,
                                   const void *W2_codes, const float *W2_scales, const void *b2, const int32_t *fill,
                                   const int32_t *capacity, void *y, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if ((st = check_blk_shape(s)) != MOE_OK) return st;
    MOE_REQUIRE(h_codes && h_scales && W2_codes && W2_scales && fill && capacity && y,
                "h, weights, fill, capacity and y must be non-NULL");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    MOE_REQUIRE_ALIGNED(h_codes, h_scales, W2_codes, W2_scales, b2, fill, capacity, y);
    hipError_t e = moe::launch_fc2_mx(s, moe::kBlkFp8, static_cast<const uint8_t *>(h_codes),
                                      reinterpret_cast<const uint8_t *>(h_scales),
                                      static_cast<const uint8_t *>(W2_codes),
                                      reinterpret_cast<const uint8_t *>(W2_scales), b2, fill, capacity, y,
                                      static_cast<int32_t>(cap_bound(s)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "block-FP8 expert fc2");
}

moe_status moe_gate_backward(const moe_shape *shape, const float *logits, const int32_t *idx, const float *dgates,
                             const int32_t *needed, double aux_coef, float *dlogits, float *aux_loss, void *ws,
                             size_t ws_bytes, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(std::isfinite(aux_coef), "aux_coef is not finite");
    MOE_REQUIRE(needed != nullptr || aux_coef == 0.0, "needed is required when aux_coef != 0");
    if (s.S > 0) MOE_REQUIRE(logits && idx && dgates && dlogits, "logits, idx, dgates and dlogits must be non-NULL");
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(logits, idx, dgates, needed, dlogits, aux_loss, ws);
    hipError_t e = moe::launch_gate_backward(s, logits, idx, dgates, needed, aux_coef, dlogits, aux_loss, ws,
                                             as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "gate backward");
}

moe_status moe_gate_weight_grad(const moe_shape *shape, const void *x, const float *dlogits, float *dWg, void *ws,
                                size_t ws_bytes, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(dWg != nullptr, "dWg is NULL");
    if (s.S > 0) MOE_REQUIRE(x && dlogits, "x and dlogits must be non-NULL");
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(x, dlogits, dWg, ws);
    hipError_t e = moe::launch_gate_weight_grad(s, x, dlogits, dWg, ws, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "gate weight gradient");
}

moe_status moe_residual_ffn(const moe_shape *shape, const void *x, const void *W1r, const void *b1r,
                            const void *W2r, const void *b2r, void *pre_r, void *h_r, void *y_r, void *ws,
                            size_t ws_bytes, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(W1r && W2r, "W1r and W2r must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && h_r && y_r, "x, h_r and y_r must be non-NULL");
    MOE_REQUIRE((b1r != nullptr) == (s.has_fc1_bias != 0), "b1r must be given iff has_fc1_bias");
    MOE_REQUIRE((b2r != nullptr) == (s.has_fc2_bias != 0), "b2r must be given iff has_fc2_bias");
    if (s.S / 128 >= 65535) return fail(MOE_EUNSUPPORTED, "S=%d too large for the dense branch's GEMM grid", s.S);
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(x, W1r, b1r, W2r, b2r, pre_r, h_r, y_r, ws);
    hipError_t e = moe::launch_residual_ffn(s, x, W1r, b1r, W2r, b2r, pre_r, h_r, y_r, static_cast<int32_t *>(ws),
                                            as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "residual dense branch");
}

moe_status moe_residual_backward(const moe_shape *shape, const void *dout, const void *x, const void *pre_r,
                                 const void *h_r, const void *W1r, const void *W2r, void *dpre_r, void *dx_r,
                                 float *dW1r, float *db1r, float *dW2r, float *db2r, void *ws, size_t ws_bytes,
                                 void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(W1r && W2r && dW1r && dW2r, "W1r, W2r, dW1r and dW2r must be non-NULL");
    if (s.S > 0)
        MOE_REQUIRE(dout && x && pre_r && h_r && dpre_r && dx_r, "dout, x, pre_r, h_r, dpre_r and dx_r must be non-NULL");
    if (s.S / 128 >= 65535) return fail(MOE_EUNSUPPORTED, "S=%d too large for the dense branch's GEMM grid", s.S);
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(dout, x, pre_r, h_r, W1r, W2r, dpre_r, dx_r, dW1r, db1r, dW2r, db2r, ws);
    hipError_t e = moe::launch_residual_bwd(s, dout, x, pre_r, h_r, W1r, W2r, dpre_r, dx_r, dW1r, db1r, dW2r, db2r,
                                            static_cast<int32_t *>(ws), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "residual dense branch backward");
}

moe_status moe_decode_residual(const moe_shape *shape, const void *y, const float *gates, const int32_t *idx,
                               const int32_t *loc, const int32_t *capacity, const void *y_r, void *out,
                               void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(capacity != nullptr, "capacity is NULL");
    if (s.S > 0) MOE_REQUIRE(y && gates && idx && loc && y_r && out, "y, gates, idx, loc, y_r and out must be non-NULL");
    MOE_REQUIRE_ALIGNED(y, gates, idx, loc, capacity, y_r, out);
    hipError_t e = moe::launch_decode(s, y, gates, idx, loc, capacity, out, false, as_stream(stream), y_r);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "decode");
}

}  // extern "C"

namespace {

struct Residual {
    const void *W1r, *b1r, *W2r, *b2r;
    void *pre_r, *h_r, *y_r;
};
// NVFP4 experts: the weights' block scales and fp32 scales (W1 and W2 are their codes).
struct Nvfp4Scales {
    const void *W1s;
    const float *W1g;
    const void *W2s;
    const float *W2g;
};

moe_status layer_forward_impl(const moe_shape *shape, const void *x, const float *logits_in, const float *Wg,
                              float *logits_out, const void *W1, const void *b1, const void *W2, const void *b2,
                              int32_t *idx, int32_t *loc, float *gates, int32_t *needed, int32_t *fill,
                              int32_t *capacity, int32_t *slot_route, void *buf, void *pre, void *h, void *y,
                              void *out, void *ws, size_t ws_bytes, const Residual *res, void *stream,
                              const Nvfp4Scales *nv = nullptr) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if (nv != nullptr) {
        if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "NVFP4 experts take bf16 tokens");
        MOE_REQUIRE(nv->W1s && nv->W1g && nv->W2s && nv->W2g, "the weights' scales and g must be non-NULL");
        MOE_REQUIRE_ALIGNED(nv->W1s, nv->W1g, nv->W2s, nv->W2g);
    }
    // with no token, empty logits may arrive as NULL
    MOE_REQUIRE(!(logits_in != nullptr && Wg != nullptr), "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(s.S == 0 || logits_in != nullptr || Wg != nullptr, "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(Wg == nullptr || logits_out != nullptr || s.S == 0, "logits_out is required with Wg");
    MOE_REQUIRE(needed && fill && capacity && buf && W1 && W2 && h && y,
                "needed, fill, capacity, buf, W1, W2, h and y must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc && gates && out, "x, idx, loc, gates and out must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    if (res != nullptr) {
        MOE_REQUIRE(res->W1r && res->W2r, "W1r and W2r must be non-NULL");
        if (s.S > 0) MOE_REQUIRE(res->h_r && res->y_r, "h_r and y_r must be non-NULL");
        MOE_REQUIRE((res->b1r != nullptr) == (s.has_fc1_bias != 0), "b1r must be given iff has_fc1_bias");
        MOE_REQUIRE((res->b2r != nullptr) == (s.has_fc2_bias != 0), "b2r must be given iff has_fc2_bias");
        if (s.S / 128 >= 65535)
            return fail(MOE_EUNSUPPORTED, "S=%d too large for the dense branch's GEMM grid", s.S);
        MOE_REQUIRE_ALIGNED(res->W1r, res->b1r, res->W2r, res->b2r, res->pre_r, res->h_r, res->y_r);
    }
    if ((st = check_forward_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill, capacity,
                        slot_route, buf, pre, h, y, out, ws);
    if (Wg != nullptr && !moe::gate_supported(s.M, s.E, s.dtype))
        return fail(MOE_EUNSUPPORTED, "gate projection tiles for M=%d, E=%d do not fit in LDS", s.M, s.E);
    hipStream_t strm = as_stream(stream);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    const float *logits = logits_in;
    hipError_t e;
    if (Wg != nullptr && s.S > 0) {
        if ((e = moe::launch_gate_project(s, x, Wg, logits_out, strm)) != hipSuccess) return hip_fail(e, "gate projection");
        logits = logits_out;
    }
    moe::RouteWs w{static_cast<int32_t *>(ws), num_tiles(s)};
    if ((e = moe::launch_route_counts(s, logits, idx, gates, needed, w, strm)) != hipSuccess)
        return hip_fail(e, "route");
    if ((e = moe::launch_assign_encode(s, x, idx, w, needed, by_factor(s), loc, fill, capacity, slot_route, buf, cmax,
                                       strm)) != hipSuccess)
        return hip_fail(e, "route assignment and encode");
    if (nv != nullptr) {
        e = moe::launch_fc1_nvfp4(s, buf, static_cast<const uint8_t *>(W1), static_cast<const uint8_t *>(nv->W1s),
                                  nv->W1g, b1, fill, capacity, pre, h, cmax, strm);
        if (e != hipSuccess) return hip_fail(e, "expert fc1 (NVFP4)");
        e = moe::launch_fc2_nvfp4(s, h, static_cast<const uint8_t *>(W2), static_cast<const uint8_t *>(nv->W2s),
                                  nv->W2g, b2, fill, capacity, y, cmax, strm);
        if (e != hipSuccess) return hip_fail(e, "expert fc2 (NVFP4)");
    } else {
        if ((e = moe::launch_fc1(s, buf, W1, b1, fill, capacity, pre, h, cmax, strm)) != hipSuccess)
            return hip_fail(e, "expert fc1");
        if ((e = moe::launch_fc2(s, h, W2, b2, fill, capacity, y, cmax, strm)) != hipSuccess)
            return hip_fail(e, "expert fc2");
    }
    // the dense branch uses the workspace after routing is done with it
    if (res != nullptr &&
        (e = moe::launch_residual_ffn(s, x, res->W1r, res->b1r, res->W2r, res->b2r, res->pre_r, res->h_r, res->y_r,
                                      static_cast<int32_t *>(ws), strm)) != hipSuccess)
        return hip_fail(e, "residual dense branch");
    if ((e = moe::launch_decode(s, y, gates, idx, loc, capacity, out, false, strm,
                                res != nullptr ? res->y_r : nullptr)) != hipSuccess)
        return hip_fail(e, "decode");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_shape *shape, const void *x, const float *logits_in, const float *Wg,
                             float *logits_out, const void *W1, const void *b1, const void *W2, const void *b2,
                             int32_t *idx, int32_t *loc, float *gates, int32_t *needed, int32_t *fill,
                             int32_t *capacity, int32_t *slot_route, void *buf, void *pre, void *h, void *y,
                             void *out, void *ws, size_t ws_bytes, void *stream) {
    return layer_forward_impl(shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill,
                              capacity, slot_route, buf, pre, h, y, out, ws, ws_bytes, nullptr, stream);
}

moe_status moe_layer_forward_nvfp4(const moe_shape *shape, const void *x, const float *logits_in, const float *Wg,
                                   float *logits_out, const void *W1_codes, const void *W1_scales, const float *W1_g,
                                   const void *b1, const void *W2_codes, const void *W2_scales, const float *W2_g,
                                   const void *b2, int32_t *idx, int32_t *loc, float *gates, int32_t *needed,
                                   int32_t *fill, int32_t *capacity, int32_t *slot_route, void *buf, void *h, void *y,
                                   void *out, void *ws, size_t ws_bytes, void *stream) {
    const Nvfp4Scales nv{W1_scales, W1_g, W2_scales, W2_g};
    return layer_forward_impl(shape, x, logits_in, Wg, logits_out, W1_codes, b1, W2_codes, b2, idx, loc, gates,
                              needed, fill, capacity, slot_route, buf, nullptr, h, y, out, ws, ws_bytes, nullptr,
                              stream, &nv);
}

moe_status moe_layer_forward_pipelined(const moe_shape *shape, const void *x, const float *logits_in,
                                       const float *Wg, float *logits_out, const void *W1, const void *b1,
                                       const void *W2, const void *b2, int32_t *idx, int32_t *loc, float *gates,
                                       int32_t *needed, int32_t *fill, int32_t *capacity, int32_t *slot_route,
                                       void *buf, void *pre, void *h, void *y, void *out, void *ws, size_t ws_bytes,
                                       int32_t chunks, void *const *streams, int32_t nstreams, void *const *events,
                                       void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    if (s.dtype != MOE_DT_BF16) return fail(MOE_EUNSUPPORTED, "the pipelined forward takes bf16 data");
    MOE_REQUIRE(chunks >= 1 && chunks <= 64, "chunks must be in [1, 64]");
    MOE_REQUIRE(nstreams >= 1 && nstreams <= 64 && streams != nullptr && events != nullptr,
                "1..64 streams and nstreams + 1 events are required");
    for (int i = 0; i < nstreams; ++i) MOE_REQUIRE(events[i] != nullptr, "events must be non-NULL");
    MOE_REQUIRE(events[nstreams] != nullptr, "events must be non-NULL");
    // everything before and after the expert FFN, checked and run by the fused forward's steps
    MOE_REQUIRE(!(logits_in != nullptr && Wg != nullptr), "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(s.S == 0 || logits_in != nullptr || Wg != nullptr, "exactly one of logits_in and Wg must be given");
    MOE_REQUIRE(Wg == nullptr || logits_out != nullptr || s.S == 0, "logits_out is required with Wg");
    MOE_REQUIRE(needed && fill && capacity && buf && W1 && W2 && h && y,
                "needed, fill, capacity, buf, W1, W2, h and y must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(x && idx && loc && gates && out, "x, idx, loc, gates and out must be non-NULL");
    MOE_REQUIRE((b1 != nullptr) == (s.has_fc1_bias != 0), "b1 must be given iff has_fc1_bias");
    MOE_REQUIRE((b2 != nullptr) == (s.has_fc2_bias != 0), "b2 must be given iff has_fc2_bias");
    if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill, capacity,
                        slot_route, buf, pre, h, y, out, ws);
    if (Wg != nullptr && !moe::gate_supported(s.M, s.E, s.dtype))
        return fail(MOE_EUNSUPPORTED, "gate projection tiles for M=%d, E=%d do not fit in LDS", s.M, s.E);
    hipStream_t strm = as_stream(stream);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    const float *logits = logits_in;
    hipError_t e;
    if (Wg != nullptr && s.S > 0) {
        if ((e = moe::launch_gate_project(s, x, Wg, logits_out, strm)) != hipSuccess) return hip_fail(e, "gate projection");
        logits = logits_out;
    }
    moe::RouteWs w{static_cast<int32_t *>(ws), num_tiles(s)};
    if ((e = moe::launch_route_counts(s, logits, idx, gates, needed, w, strm)) != hipSuccess)
        return hip_fail(e, "route");
    if ((e = moe::launch_assign_encode(s, x, idx, w, needed, by_factor(s), loc, fill, capacity, slot_route, buf, cmax,
                                       strm)) != hipSuccess)
        return hip_fail(e, "route assignment and encode");
    auto ev = [&](int i) { return reinterpret_cast<hipEvent_t>(events[i]); };
    if ((e = hipEventRecord(ev(0), strm)) != hipSuccess) return hip_fail(e, "event record");
    for (int i = 0; i < nstreams; ++i)
        if ((e = hipStreamWaitEvent(as_stream(streams[i]), ev(0), 0)) != hipSuccess) return hip_fail(e, "stream wait");
    const int32_t width = (cmax + chunks - 1) / chunks;
    for (int c = 0; c < chunks && c * width < cmax; ++c) {
        const int32_t a = c * width, b = std::min(cmax, a + width);
        if ((e = moe::launch_ffn_window(s, buf, W1, b1, W2, b2, fill, capacity, pre, h, y, cmax, a, b,
                                        as_stream(streams[c % nstreams]))) != hipSuccess)
            return hip_fail(e, "expert ffn window");
    }
    for (int i = 0; i < nstreams; ++i) {
        if ((e = hipEventRecord(ev(i + 1), as_stream(streams[i]))) != hipSuccess) return hip_fail(e, "event record");
        if ((e = hipStreamWaitEvent(strm, ev(i + 1), 0)) != hipSuccess) return hip_fail(e, "stream wait");
    }
    if ((e = moe::launch_decode(s, y, gates, idx, loc, capacity, out, false, strm)) != hipSuccess)
        return hip_fail(e, "decode");
    return MOE_OK;
}

moe_status moe_residual_layer_forward(const moe_shape *shape, const void *x, const float *logits_in,
                                      const float *Wg, float *logits_out, const void *W1, const void *b1,
                                      const void *W2, const void *b2, const void *W1r, const void *b1r,
                                      const void *W2r, const void *b2r, int32_t *idx, int32_t *loc, float *gates,
                                      int32_t *needed, int32_t *fill, int32_t *capacity, int32_t *slot_route,
                                      void *buf, void *pre, void *h, void *y, void *pre_r, void *h_r, void *y_r,
                                      void *out, void *ws, size_t ws_bytes, void *stream) {
    const Residual res{W1r, b1r, W2r, b2r, pre_r, h_r, y_r};
    return layer_forward_impl(shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill,
                              capacity, slot_route, buf, pre, h, y, out, ws, ws_bytes, &res, stream);
}

moe_status moe_decode_backward(const moe_shape *shape, const void *dout, const void *y, const float *gates,
                               const int32_t *idx, const int32_t *loc, const int32_t *capacity, void *dy,
                               float *dgates, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(capacity != nullptr, "capacity is NULL");
    if (s.S > 0) MOE_REQUIRE(dout && y && gates && idx && loc && dy && dgates,
                             "dout, y, gates, idx, loc, dy and dgates must be non-NULL");
    MOE_REQUIRE_ALIGNED(dout, y, gates, idx, loc, capacity, dy, dgates);
    hipError_t e = moe::launch_decode_bwd(s, dout, y, gates, idx, loc, capacity, dy, dgates, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "decode backward");
}

moe_status moe_expert_fc2_backward_data(const moe_shape *shape, const void *dy, const void *W2, const void *pre,
                                        const int32_t *fill, const int32_t *capacity, void *dpre, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(dy && W2 && pre && fill && capacity && dpre, "dy, W2, pre, fill, capacity and dpre must be non-NULL");
    MOE_REQUIRE_ALIGNED(dy, W2, pre, fill, capacity, dpre);
    hipError_t e = moe::launch_fc2_bwd_data(*shape, dy, W2, pre, fill, capacity, dpre,
                                            static_cast<int32_t>(cap_bound(*shape)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fc2 backward (data)");
}

moe_status moe_expert_fc2_weight_grad(const moe_shape *shape, const void *dy, const void *h, const int32_t *fill,
                                      const int32_t *capacity, float *dW2, float *db2, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(dy && h && fill && capacity && dW2, "dy, h, fill, capacity and dW2 must be non-NULL");
    MOE_REQUIRE_ALIGNED(dy, h, fill, capacity, dW2, db2);
    hipError_t e = moe::launch_fc2_wgrad(*shape, dy, h, fill, capacity, dW2, db2,
                                         static_cast<int32_t>(cap_bound(*shape)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fc2 weight gradient");
}

moe_status moe_expert_fc1_backward_data(const moe_shape *shape, const void *dpre, const void *W1, const int32_t *fill,
                                        const int32_t *capacity, void *dbuf, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(dpre && W1 && fill && capacity && dbuf, "dpre, W1, fill, capacity and dbuf must be non-NULL");
    MOE_REQUIRE_ALIGNED(dpre, W1, fill, capacity, dbuf);
    hipError_t e = moe::launch_fc1_bwd_data(*shape, dpre, W1, fill, capacity, dbuf,
                                            static_cast<int32_t>(cap_bound(*shape)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fc1 backward (data)");
}

moe_status moe_expert_fc1_weight_grad(const moe_shape *shape, const void *dpre, const void *buf, const int32_t *fill,
                                      const int32_t *capacity, float *dW1, float *db1, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(dpre && buf && fill && capacity && dW1, "dpre, buf, fill, capacity and dW1 must be non-NULL");
    MOE_REQUIRE_ALIGNED(dpre, buf, fill, capacity, dW1, db1);
    hipError_t e = moe::launch_fc1_wgrad(*shape, dpre, buf, fill, capacity, dW1, db1,
                                         static_cast<int32_t>(cap_bound(*shape)), as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fc1 weight gradient");
}

moe_status moe_encode_backward(const moe_shape *shape, const void *dbuf, const int32_t *idx, const int32_t *loc,
                               const int32_t *capacity, void *dx, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(capacity != nullptr, "capacity is NULL");
    if (s.S > 0) MOE_REQUIRE(dbuf && idx && loc && dx, "dbuf, idx, loc and dx must be non-NULL");
    MOE_REQUIRE_ALIGNED(dbuf, idx, loc, capacity, dx);
    hipError_t e = moe::launch_decode(s, dbuf, nullptr, idx, loc, capacity, dx, true, as_stream(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "encode backward");
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Residual-MoE's dense branch in the layer backward: its forward tensors, weights and
// gradient outputs.
struct ResidualGrad {
    const void *W1r, *W2r, *pre_r, *h_r;
    void *dpre_r, *dx_r;
    float *dW1r, *db1r, *dW2r, *db2r;
};

moe_status layer_backward_impl(const moe_shape *shape, const void *dout, const void *buf, const void *pre,
                               const void *h, const void *y, const float *gates, const int32_t *idx,
                               const int32_t *loc, const int32_t *fill, const int32_t *capacity, const void *W1,
                               const void *W2, void *dy, void *dpre, void *dbuf, void *dx, float *dW1, float *db1,
                               float *dW2, float *db2, float *dgates, const float *logits, const int32_t *needed,
                               double aux_coef, const void *x, const float *Wg, float *dlogits, float *dWg,
                               float *aux_loss, void *ws, size_t ws_bytes, const ResidualGrad *res, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape &s = *shape;
    MOE_REQUIRE(buf && pre && h && y && fill && capacity && W1 && W2 && dy && dpre && dbuf && dW1 && dW2,
                "buf, pre, h, y, fill, capacity, W1, W2, dy, dpre, dbuf, dW1 and dW2 must be non-NULL");
    if (s.S > 0) MOE_REQUIRE(dout && gates && idx && loc && dx && dgates, "dout, gates, idx, loc, dx and dgates must be non-NULL");
    // the gate backward runs when any of its inputs or outputs is given
    const bool gate = logits != nullptr || dlogits != nullptr || dWg != nullptr || aux_loss != nullptr;
    if (gate) {
        MOE_REQUIRE(std::isfinite(aux_coef), "aux_coef is not finite");
        MOE_REQUIRE(needed != nullptr || aux_coef == 0.0, "needed is required when aux_coef != 0");
        if (s.S > 0) MOE_REQUIRE(logits && dlogits, "the gate backward needs logits and dlogits");
        MOE_REQUIRE((Wg != nullptr) == (dWg != nullptr), "Wg and dWg go together");
        if (s.S > 0 && Wg != nullptr) MOE_REQUIRE(x != nullptr, "x is required with Wg");
    } else {
        MOE_REQUIRE(Wg == nullptr, "Wg needs the gate backward (logits, dlogits, dWg)");
    }
    if (res != nullptr) {
        MOE_REQUIRE(res->W1r && res->W2r && res->dW1r && res->dW2r, "W1r, W2r, dW1r and dW2r must be non-NULL");
        if (s.S > 0)
            MOE_REQUIRE(x && res->pre_r && res->h_r && res->dpre_r && res->dx_r,
                        "x, pre_r, h_r, dpre_r and dx_r must be non-NULL");
        MOE_REQUIRE(res->dx_r != dx || s.S == 0, "dx_r and dx must be different buffers");
        if (s.S / 128 >= 65535)
            return fail(MOE_EUNSUPPORTED, "S=%d too large for the dense branch's GEMM grid", s.S);
        MOE_REQUIRE_ALIGNED(res->W1r, res->W2r, res->pre_r, res->h_r, res->dpre_r, res->dx_r, res->dW1r, res->db1r,
                            res->dW2r, res->db2r);
    }
    if (gate || res != nullptr)
        if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
    MOE_REQUIRE_ALIGNED(dout, buf, pre, h, y, gates, idx, loc, fill, capacity, W1, W2, dy, dpre, dbuf, dx, dW1, db1,
                        dW2, db2, dgates, logits, needed, x, Wg, dlogits, dWg, aux_loss, ws);
    hipStream_t strm = as_stream(stream);
    const int32_t cmax = static_cast<int32_t>(cap_bound(s));
    hipError_t e;
    // the dense branch first: its two row counts in the workspace are read before the
    // gate backward reuses the workspace (stream order)
    if (res != nullptr &&
        (e = moe::launch_residual_bwd(s, dout, x, res->pre_r, res->h_r, res->W1r, res->W2r, res->dpre_r, res->dx_r,
                                      res->dW1r, res->db1r, res->dW2r, res->db2r, static_cast<int32_t *>(ws),
                                      strm)) != hipSuccess)
        return hip_fail(e, "residual dense branch backward");
    if ((e = moe::launch_decode_bwd(s, dout, y, gates, idx, loc, capacity, dy, dgates, strm)) != hipSuccess)
        return hip_fail(e, "decode backward");
    if (gate) {
        if ((e = moe::launch_gate_backward(s, logits, idx, dgates, needed, aux_coef, dlogits, aux_loss, ws, strm)) !=
            hipSuccess)
            return hip_fail(e, "gate backward");
        if (Wg != nullptr && (e = moe::launch_gate_weight_grad(s, x, dlogits, dWg, ws, strm)) != hipSuccess)
            return hip_fail(e, "gate weight gradient");
    }
    if ((e = moe::launch_expert_ffn_bwd(s, buf, pre, h, W1, W2, fill, capacity, dy, dpre, dbuf, dW1, db1, dW2, db2,
                                        cmax, strm)) != hipSuccess)
        return hip_fail(e, "expert ffn backward");
    const void *dxres = res != nullptr ? res->dx_r : nullptr;
    if (gate && Wg != nullptr)
        e = moe::launch_gate_dx(s, dbuf, idx, loc, capacity, dlogits, Wg, dx, strm, dxres);
    else
        e = moe::launch_decode(s, dbuf, nullptr, idx, loc, capacity, dx, true, strm, dxres);
    if (e != hipSuccess) return hip_fail(e, "encode backward");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_backward(const moe_shape *shape, const void *dout, const void *buf, const void *pre,
                              const void *h, const void *y, const float *gates, const int32_t *idx,
                              const int32_t *loc, const int32_t *fill, const int32_t *capacity, const void *W1,
                              const void *W2, void *dy, void *dpre, void *dbuf, void *dx, float *dW1, float *db1,
                              float *dW2, float *db2, float *dgates, const float *logits, const int32_t *needed,
                              double aux_coef, const void *x, const float *Wg, float *dlogits, float *dWg,
                              float *aux_loss, void *ws, size_t ws_bytes, void *stream) {
    return layer_backward_impl(shape, dout, buf, pre, h, y, gates, idx, loc, fill, capacity, W1, W2, dy, dpre, dbuf,
                               dx, dW1, db1, dW2, db2, dgates, logits, needed, aux_coef, x, Wg, dlogits, dWg, aux_loss,
                               ws, ws_bytes, nullptr, stream);
}

moe_status moe_residual_layer_backward(const moe_shape *shape, const void *dout, const void *buf, const void *pre,
                                       const void *h, const void *y, const float *gates, const int32_t *idx,
                                       const int32_t *loc, const int32_t *fill, const int32_t *capacity,
                                       const void *W1, const void *W2, void *dy, void *dpre, void *dbuf, void *dx,
                                       float *dW1, float *db1, float *dW2, float *db2, float *dgates,
                                       const float *logits, const int32_t *needed, double aux_coef, const void *x,
                                       const float *Wg, float *dlogits, float *dWg, float *aux_loss,
                                       const void *W1r, const void *W2r, const void *pre_r, const void *h_r,
                                       void *dpre_r, void *dx_r, float *dW1r, float *db1r, float *dW2r, float *db2r,
                                       void *ws, size_t ws_bytes, void *stream) {
    const ResidualGrad res{W1r, W2r, pre_r, h_r, dpre_r, dx_r, dW1r, db1r, dW2r, db2r};
    return layer_backward_impl(shape, dout, buf, pre, h, y, gates, idx, loc, fill, capacity, W1, W2, dy, dpre, dbuf,
                               dx, dW1, db1, dW2, db2, dgates, logits, needed, aux_coef, x, Wg, dlogits, dWg, aux_loss,
                               ws, ws_bytes, &res, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- the forward without allocation
// moe_layer_forward_noalloc keeps routing's workspace in this array instead of a
// caller buffer. Each GPU the library runs on holds its own copy of it, at its own
// address, until the process ends; every call on a GPU shares that GPU's copy.
// Routing writes every count it later reads, so nothing in it has to start at zero.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device address of `scratch` on the device of `stream` (the current device for
// NULL), looked up once per device with that device current. Host code uses only
// this address: the array's name is a host-side stand-in, not a device pointer.
moe_status scratch_address(hipStream_t stream, void **addr) {
    int dev = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "device of the stream");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "current device");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "set device");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
        if (p == nullptr) return fail(MOE_EHIP, "address of the static scratch is NULL");
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_shape *shape, const void *x, const float *logits_in, const float *Wg,
                                     float *logits_out, const void *W1, const void *b1, const void *W2,
                                     const void *b2, int32_t *idx, int32_t *loc, float *gates, int32_t *needed,
                                     int32_t *fill, int32_t *capacity, int32_t *slot_route, void *buf, void *pre,
                                     void *h, void *y, void *out, void *stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    const size_t need = forward_ws_bytes(*shape);
    if (need > kNoAllocScratchBytes)
        return fail(MOE_EUNSUPPORTED,
                    "routing needs %zu bytes of workspace (E*k*ceil(S/64) counts), above the %zu-byte static scratch "
                    "of moe_layer_forward_noalloc: use moe_layer_forward with a workspace",
                    need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_address(as_stream(stream), &ws)) != MOE_OK) return st;
    return layer_forward_impl(shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill,
                              capacity, slot_route, buf, pre, h, y, out, ws, kNoAllocScratchBytes, nullptr, stream);
}

}  // extern "C"
