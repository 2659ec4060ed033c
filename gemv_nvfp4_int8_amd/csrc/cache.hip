// cache.hip -- derived-weight cache: a weight is requantised on first use and
// the result is kept for the life of the cache, keyed by the source weight's
// device address (dispatch_proj_rowwise.rs, requant_weight_rowwise_fp8_cached
// with its DerivedWeights cache; gemm_dense_int8.rs, requant_w_nvfp4_int8,
// whose int8 copy is made once per weight).
//
// Host code only.  The derivation itself is the stateless entry point's
// kernel, enqueued on the caller's stream; the cache owns the derived device
// buffers (hipMalloc on a miss, hipFree on evict / destroy).  A derivation
// has no transient buffer, so nothing waits on the host: each entry records
// an event after its launch, and every hit makes the caller's stream wait for
// that event, so a derived weight is safe to use from any stream.
#include <hip/hip_runtime.h>

#include <initializer_list>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/qproj.h"

struct qp_cache {
    struct Entry {
        void *w = nullptr;          // derived weight (device)
        void *s = nullptr;          // derived scales (device)
        uint64_t bytes = 0;
        uint32_t n = 0, k = 0;
        uint32_t scale2_bits = 0;   // the NVFP4 scale2 the int8 copy was made with
        hipEvent_t ready = nullptr; // recorded after the derivation's launch
    };
    std::mutex mu;
    std::map<std::pair<int, uintptr_t>, Entry> map;   // (derivation, source) -> entry
    uint64_t bytes = 0;
};

namespace {

enum Derivation { ROWWISE_FP8 = 1, INT8_BLOCK32 = 2 };

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_ptrs(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!p)
            return QP_ERR_NULL;
    for (const void *p : ps)
        if (!aligned16(p))
            return QP_ERR_ALIGN;
    return QP_OK;
}

inline int check2(const void *a, const void *b) { return check_ptrs({a, b}); }

inline bool fits(uint64_t rows, uint64_t cols) { return rows * cols < (1ull << 31); }

void release(qp_cache::Entry &e)
{
    (void)hipFree(e.w);
    (void)hipFree(e.s);
    if (e.ready)
        (void)hipEventDestroy(e.ready);
}

uint32_t bits_of(float f)
{
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    return u;
}

// Look up (kind, src); on a miss allocate wbytes + sbytes, run launch(w, s)
// on the stream and record the entry.  The whole miss holds the lock, so a
// weight is derived once even when several threads ask for it together.
template <class Launch>
int get_or_derive(qp_cache *c, int kind, const void *src, uint32_t n, uint32_t k,
                  uint32_t scale2_bits, uint64_t wbytes, uint64_t sbytes, hipStream_t st,
                  Launch launch, void **w_out, void **s_out)
{
    std::lock_guard<std::mutex> lock(c->mu);
    auto key = std::make_pair(kind, reinterpret_cast<uintptr_t>(src));
    auto it = c->map.find(key);
    if (it != c->map.end()) {
        const qp_cache::Entry &e = it->second;
        if (e.n != n || e.k != k || e.scale2_bits != scale2_bits)
            return QP_ERR_SHAPE;            // the address now holds a different weight
        if (hipStreamWaitEvent(st, e.ready, 0) != hipSuccess)
            return QP_ERR_HIP;
        *w_out = e.w;
        *s_out = e.s;
        return QP_OK;
    }
    qp_cache::Entry e;
    e.n = n;
    e.k = k;
    e.scale2_bits = scale2_bits;
    e.bytes = wbytes + sbytes;
    if (hipMalloc(&e.w, wbytes) != hipSuccess || hipMalloc(&e.s, sbytes) != hipSuccess) {
        release(e);
        return QP_ERR_ALLOC;
    }
    if (hipEventCreateWithFlags(&e.ready, hipEventDisableTiming) != hipSuccess) {
        e.ready = nullptr;
        release(e);
        return QP_ERR_HIP;
    }
    if (int rc = launch(e.w, e.s)) {
        release(e);
        return rc;
    }
    if (hipEventRecord(e.ready, st) != hipSuccess) {
        release(e);
        return QP_ERR_HIP;
    }
    c->map.emplace(key, e);
    c->bytes += e.bytes;
    *w_out = e.w;
    *s_out = e.s;
    return QP_OK;
}

} // namespace

extern "C" {

int qproj_cache_create(qp_cache **cache)
{
    if (!cache)
        return QP_ERR_NULL;
    *cache = new qp_cache();
    return QP_OK;
}

int qproj_cache_destroy(qp_cache *cache)
{
    if (!cache)
        return QP_ERR_NULL;
    {
        std::lock_guard<std::mutex> lock(cache->mu);
        for (auto &kv : cache->map)
            release(kv.second);
    }
    delete cache;
    return QP_OK;
}

int qproj_cache_evict(qp_cache *cache, const void *weight)
{
    if (!cache || !weight)
        return QP_ERR_NULL;
    std::lock_guard<std::mutex> lock(cache->mu);
    for (int kind : {ROWWISE_FP8, INT8_BLOCK32}) {
        auto it = cache->map.find(std::make_pair(kind, reinterpret_cast<uintptr_t>(weight)));
        if (it != cache->map.end()) {
            cache->bytes -= it->second.bytes;
            release(it->second);
            cache->map.erase(it);
        }
    }
    return QP_OK;
}

int qproj_cache_stats(qp_cache *cache, uint64_t *entries, uint64_t *bytes)
{
    if (!cache || !entries || !bytes)
        return QP_ERR_NULL;
    std::lock_guard<std::mutex> lock(cache->mu);
    *entries = cache->map.size();
    *bytes = cache->bytes;
    return QP_OK;
}

int requant_w_blockfp8_rowwise_cached(qp_cache *cache, int fmt, const uint8_t *w,
                                      const float *scale, uint32_t n, uint32_t k,
                                      const uint8_t **w_rowwise, const float **w_rowwise_scale,
                                      void *stream)
{
    if (!cache || !w_rowwise || !w_rowwise_scale)
        return QP_ERR_NULL;
    if (fmt == QP_FP8_PER_ROW) {
        // Already row-wise: the caller's own buffers, no work and no entry.
        return requant_w_blockfp8_rowwise(fmt, w, scale, nullptr, nullptr, w_rowwise,
                                          w_rowwise_scale, n, k, stream);
    }
    if (fmt != QP_FP8_BLOCK128)
        return QP_ERR_FORMAT;
    if (int e = check2(w, scale))
        return e;
    if (n == 0 || k == 0 || n % 128 != 0 || k % 128 != 0 || !fits(n, k))
        return QP_ERR_SHAPE;
    void *wq = nullptr, *sq = nullptr;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int rc = get_or_derive(
        cache, ROWWISE_FP8, w, n, k, 0, (uint64_t)n * k, (uint64_t)n * 4, st,
        [&](void *dw, void *ds) {
            const uint8_t *r0;
            const float *r1;
            return requant_w_blockfp8_rowwise(fmt, w, scale, static_cast<uint8_t *>(dw),
                                              static_cast<float *>(ds), &r0, &r1, n, k,
                                              stream);
        },
        &wq, &sq);
    if (rc)
        return rc;
    *w_rowwise = static_cast<const uint8_t *>(wq);
    *w_rowwise_scale = static_cast<const float *>(sq);
    return QP_OK;
}

int requant_w_nvfp4_int8_cached(qp_cache *cache, const uint8_t *w_packed,
                                const uint8_t *w_e4m3, float scale2, uint32_t n, uint32_t k,
                                const int8_t **w_i8, const float **w_scale, void *stream)
{
    if (!cache || !w_i8 || !w_scale)
        return QP_ERR_NULL;
    if (int e = check2(w_packed, w_e4m3))
        return e;
    if (n == 0 || k == 0 || k % 32 != 0 || !fits(n, k))
        return QP_ERR_SHAPE;
    void *wq = nullptr, *sq = nullptr;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int rc = get_or_derive(
        cache, INT8_BLOCK32, w_packed, n, k, bits_of(scale2), (uint64_t)n * k,
        (uint64_t)n * (k / 32) * 4, st,
        [&](void *dw, void *ds) {
            return requant_w_nvfp4_int8(w_packed, w_e4m3, scale2, static_cast<int8_t *>(dw),
                                        static_cast<float *>(ds), n, k, stream);
        },
        &wq, &sq);
    if (rc)
        return rc;
    *w_i8 = static_cast<const int8_t *>(wq);
    *w_scale = static_cast<const float *>(sq);
    return QP_OK;
}

int fp8_rowwise_proj_cached(qp_cache *cache, int fmt, const uint8_t *w, const float *w_scale,
                            const uint16_t *act, uint8_t *act_q, float *act_scale,
                            uint16_t *out, uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    // the projection's own arguments first, so a bad call derives nothing
    if (int e = check_ptrs({act, act_q, act_scale, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 16 != 0 || !fits(m, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    const uint8_t *wq = nullptr;
    const float *ws = nullptr;
    if (int e = requant_w_blockfp8_rowwise_cached(cache, fmt, w, w_scale, n, k, &wq, &ws, stream))
        return e;
    if (int e = quant_rowwise_fp8(act, act_q, act_scale, m, k, stream))
        return e;
    return fp8_gemm_rowscale(act_q, act_scale, wq, ws, out, m, n, k, stream);
}

int int8_w4a8_prefill_cached(qp_cache *cache, const uint16_t *a_bf16, const uint8_t *w_packed,
                             const uint8_t *w_e4m3, float scale2, int8_t *a_i8_scratch,
                             float *a_scale_scratch, uint16_t *out, uint32_t m, uint32_t n,
                             uint32_t k, void *stream)
{
    if (int e = check_ptrs({a_bf16, a_i8_scratch, a_scale_scratch, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || !fits(m, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    const int8_t *wq = nullptr;
    const float *ws = nullptr;
    if (int e = requant_w_nvfp4_int8_cached(cache, w_packed, w_e4m3, scale2, n, k, &wq, &ws,
                                            stream))
        return e;
    return int8_w4a8_prefill(a_bf16, wq, ws, a_i8_scratch, a_scale_scratch, out, m, n, k,
                             stream);
}

} // extern "C"
