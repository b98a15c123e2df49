// dsa_abi.hip -- the C ABI of include/dsa.h: host-side validation, workspace
// carve-up and launch composition. Every refusal happens here, before any HIP
// call, in the manner of the glm5next_dsa/layer.rs source page (`decode_k`
// bails out on lockstep, row-count and metadata mismatches before touching the
// device; `indexer_forward` checks room before any write).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "dsa.h"
#include "dsa_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptr(const void *p, const char *name)
{
    if (!p)
        return fail(DSA_EINVAL, "%s is NULL", name);
    if (!aligned16(p))
        return fail(DSA_EINVAL, "%s is not 16-byte aligned", name);
    return DSA_OK;
}

int check_shape(const dsa_shape *sh, dsa::LaunchShape *ls)
{
    if (!sh)
        return fail(DSA_EINVAL, "shape is NULL");
    if (sh->num_seqs < 1 || sh->rows_per_seq < 1 || sh->num_heads < 1 || sh->latent_dim < 1 ||
        sh->index_heads < 1 || sh->index_dim < 1 || sh->top_k < 1 || sh->page_size < 1 ||
        sh->max_len < 1 || sh->k_capacity < 1 || sh->max_blocks_per_seq < 1 || sh->num_pages < 1)
        return fail(DSA_EINVAL, "every dsa_shape field must be positive");
    if (sh->rows_per_seq > dsa::kMaxRowsPerSeq)
        return fail(DSA_EUNSUPPORTED, "rows_per_seq %d outside [1, %d]", sh->rows_per_seq,
                    dsa::kMaxRowsPerSeq);
    if (sh->latent_dim != 512)
        return fail(DSA_EUNSUPPORTED, "latent_dim %d: only 512 is supported", sh->latent_dim);
    if (sh->num_heads > 128)
        return fail(DSA_EUNSUPPORTED, "num_heads %d above 128", sh->num_heads);
    if (sh->index_heads > 32)
        return fail(DSA_EUNSUPPORTED, "index_heads %d above 32", sh->index_heads);
    if (sh->index_dim != 64 && sh->index_dim != 128)
        return fail(DSA_EUNSUPPORTED, "index_dim %d: only 64 and 128 are supported", sh->index_dim);
    if (sh->top_k > 16384)
        return fail(DSA_EUNSUPPORTED, "top_k %d above 16384", sh->top_k);
    if (sh->max_len > (1 << 22))
        return fail(DSA_ERANGE, "max_len %d above 4194304", sh->max_len);
    if (sh->k_capacity < sh->max_len)
        return fail(DSA_ERANGE, "k_capacity %d below max_len %d", sh->k_capacity, sh->max_len);
    if ((int64_t)sh->max_blocks_per_seq * sh->page_size < sh->max_len)
        return fail(DSA_ERANGE,
                    "block table too short: %d entries x page_size %d cannot address max_len %d",
                    sh->max_blocks_per_seq, sh->page_size, sh->max_len);
    if ((int64_t)sh->num_pages * sh->page_size > 0x7FFFFFFF)
        return fail(DSA_ERANGE, "num_pages x page_size above 2^31 - 1 latent rows");
    const int64_t rows = (int64_t)sh->num_seqs * sh->rows_per_seq;
    if (rows > 65535)
        return fail(DSA_EUNSUPPORTED, "%lld rows above 65535", (long long)rows);
    ls->num_seqs = sh->num_seqs;
    ls->rows_per_seq = sh->rows_per_seq;
    ls->num_rows = (int)rows;
    ls->num_heads = sh->num_heads;
    ls->latent_dim = sh->latent_dim;
    ls->index_heads = sh->index_heads;
    ls->index_dim = sh->index_dim;
    ls->top_k = sh->top_k;
    ls->page_size = sh->page_size;
    ls->max_len = sh->max_len;
    ls->k_capacity = sh->k_capacity;
    ls->max_blocks = sh->max_blocks_per_seq;
    ls->num_pages = sh->num_pages;
    return DSA_OK;
}

int check_ws(const void *ws, size_t ws_bytes, const dsa::Workspace &wl)
{
    if (check_ptr(ws, "ws") != DSA_OK)
        return fail(DSA_EWORKSPACE, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < wl.total)
        return fail(DSA_EWORKSPACE, "workspace of %zu bytes is below the %zu this shape needs",
                    ws_bytes, wl.total);
    return DSA_OK;
}

int launched(int rc, const char *what)
{
    if (rc != 0)
        return fail(DSA_ELAUNCH, "HIP refused the %s launch: %s", what,
                    hipGetErrorString(hipGetLastError()));
    return DSA_OK;
}

constexpr int kMaxPoolTokens = 1024; // kp above this is refused

// The pooled selection's shapes and workspace: the token shape's selector run
// on pools (max_len = max(1, max_len / kp) pools, top_k = select_k pools),
// then per-row pool counts and the selected pools.
struct PooledLayout {
    dsa::LaunchShape ls_pool;
    dsa::Workspace wl;
    size_t pool_lens, sel_pools, masked, total;
    int max_len; // the token ceiling
    bool any_pool;
};

int pooled_layout(const dsa_shape *shape, int32_t kp, PooledLayout *pl)
{
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if (kp < 1 || kp > kMaxPoolTokens)
        return fail(DSA_EUNSUPPORTED, "pool size %d outside [1, %d]", kp, kMaxPoolTokens);
    pl->max_len = ls.max_len;
    pl->any_pool = ls.max_len >= kp;
    pl->ls_pool = ls;
    pl->ls_pool.max_len = ls.max_len / kp > 0 ? ls.max_len / kp : 1;
    pl->wl = dsa::workspace_layout(pl->ls_pool);
    size_t off = pl->wl.total;
    pl->pool_lens = off;
    off = align256(off + (size_t)ls.num_rows * sizeof(int32_t));
    pl->sel_pools = off;
    off = align256(off + (size_t)ls.num_rows * ls.top_k * sizeof(int32_t));
    pl->masked = off; // pool scores with the incomplete pools at -inf (pool_valid given)
    off = align256(off + (size_t)ls.num_rows * (size_t)dsa::score_stride(pl->ls_pool) * sizeof(float));
    pl->total = off;
    return DSA_OK;
}

} // namespace

static_assert(DSA_SELECT_DIRECT_MAX == dsa::kSelDirectMax, "header and kernels agree");

namespace dsa {

Workspace workspace_layout(const LaunchShape &ls)
{
    Workspace w{};
    const size_t R = (size_t)ls.num_rows;
    const size_t stride = (size_t)score_stride(ls);
    const size_t nch = (size_t)att_chunks(ls);
    const size_t hgc = (size_t)att_head_groups(ls);
    size_t off = 0;
    w.cand = off;
    off = align256(off + R * stride * 8);
    w.bitmap = off;
    off = align256(off + R * (stride / 32) * 4);
    w.cnt = off;
    off = align256(off + R * (size_t)dsa::sel_slices(ls) * 4);
    w.gm4 = off;
    off = align256(off + R * (stride / 4) * 4);
    w.gm32 = off;
    off = align256(off + R * (stride / 32) * 4);
    w.part_ml = off;
    w.part_o = off;
    if (nch > 1) {
        off = align256(off + R * hgc * nch * kAttHeads * 2 * sizeof(float));
        w.part_o = off;
        off = align256(off + R * hgc * nch * kAttHeads * 512 * sizeof(uint16_t)); // bf16 O
    }
    w.total = off;
    return w;
}

} // namespace dsa

namespace {

// Library-owned workspace of dsa_decode_k_noalloc: one per device, held until
// the process ends. Host code never passes `scratch` itself to a kernel or a
// copy (on the host the name is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current). Returns DSA_OK or a refusal.
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(DSA_ELAUNCH, "no usable current device (hipGetDevice gave %d)", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(DSA_ELAUNCH, "hipGetSymbolAddress of the scratch array failed on device %d: %s",
                        dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

} // namespace

extern "C" {

size_t dsa_workspace_bytes(const dsa_shape *shape)
{
    dsa::LaunchShape ls;
    if (check_shape(shape, &ls) != DSA_OK)
        return 0;
    return dsa::workspace_layout(ls).total;
}

const char *dsa_last_error(void) { return g_err; }

size_t dsa_score_stride(const dsa_shape *shape)
{
    dsa::LaunchShape ls;
    if (check_shape(shape, &ls) != DSA_OK)
        return 0;
    return (size_t)dsa::score_stride(ls);
}

size_t dsa_pooled_workspace_bytes(const dsa_shape *shape, int32_t kp)
{
    PooledLayout pl;
    if (pooled_layout(shape, kp, &pl) != DSA_OK)
        return 0;
    return pl.total;
}

size_t dsa_pool_score_stride(const dsa_shape *shape, int32_t kp)
{
    PooledLayout pl;
    if (pooled_layout(shape, kp, &pl) != DSA_OK)
        return 0;
    return (size_t)dsa::score_stride(pl.ls_pool);
}

int dsa_topk_select_pooled(const dsa_shape *shape, int32_t kp, const float *pool_scores,
                           const uint8_t *pool_valid, const int32_t *seq_lens, int32_t *sel,
                           void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    PooledLayout pl;
    int rc;
    if ((rc = pooled_layout(shape, kp, &pl)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(pool_scores, "pool_scores")) || (rc = check_ptr(seq_lens, "seq_lens")) ||
        (rc = check_ptr(sel, "sel")))
        return rc;
    if (pool_valid != nullptr && ((uintptr_t)pool_valid % 16) != 0)
        return fail(DSA_EINVAL, "pool_valid is not 16-byte aligned");
    if (check_ptr(ws, "ws") != DSA_OK)
        return fail(DSA_EWORKSPACE, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < pl.total)
        return fail(DSA_EWORKSPACE, "workspace of %zu bytes is below the %zu this shape needs",
                    ws_bytes, pl.total);
    return launched(dsa::launch_select_pooled(pl.ls_pool, pl.max_len, kp, pool_scores, pool_valid,
                                              seq_lens, sel, (char *)ws, pl.wl, pl.pool_lens,
                                              pl.sel_pools, pl.masked, pl.any_pool,
                                              (hipStream_t)stream),
                    "select_pooled");
}

size_t dsa_bt_entries_needed(size_t seq_len, size_t k, size_t block_size)
{
    return (seq_len + k) / (block_size ? block_size : 1) + 2;
}

int dsa_index_scores(const dsa_shape *shape, const void *q_idx, const float *w,
                     const void *k_normed, const int32_t *seq_lens, float *scores, void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(q_idx, "q_idx")) || (rc = check_ptr(w, "w")) ||
        (rc = check_ptr(k_normed, "k_normed")) || (rc = check_ptr(seq_lens, "seq_lens")) ||
        (rc = check_ptr(scores, "scores")))
        return rc;
    return launched(dsa::launch_index_scores(ls, (const uint16_t *)q_idx, w,
                                             (const uint16_t *)k_normed, seq_lens, scores,
                                             nullptr, nullptr, (hipStream_t)stream),
                    "index_scores");
}

int dsa_topk_select(const dsa_shape *shape, const float *scores, const int32_t *seq_lens,
                    int32_t *sel, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(scores, "scores")) || (rc = check_ptr(seq_lens, "seq_lens")) ||
        (rc = check_ptr(sel, "sel")))
        return rc;
    const dsa::Workspace wl = dsa::workspace_layout(ls);
    if ((rc = check_ws(ws, ws_bytes, wl)) != DSA_OK)
        return rc;
    return launched(dsa::launch_select(ls, scores, seq_lens, sel, (char *)ws, wl, false,
                                       (hipStream_t)stream),
                    "select");
}

int dsa_mla_decode(const dsa_shape *shape, const void *q, const uint8_t *kv_cache,
                   const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                   float kv_scale, float sm_scale, void *out, void *ws, size_t ws_bytes,
                   void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(q, "q")) || (rc = check_ptr(kv_cache, "kv_cache")) ||
        (rc = check_ptr(block_tables, "block_tables")) || (rc = check_ptr(seq_lens, "seq_lens")) ||
        (rc = check_ptr(sel, "sel")) || (rc = check_ptr(out, "out")))
        return rc;
    if (!(kv_scale > 0.0f) || !(sm_scale > 0.0f) || kv_scale == __builtin_huge_valf() ||
        sm_scale == __builtin_huge_valf())
        return fail(DSA_EINVAL, "kv_scale and sm_scale must be positive and finite");
    const dsa::Workspace wl = dsa::workspace_layout(ls);
    if ((rc = check_ws(ws, ws_bytes, wl)) != DSA_OK)
        return rc;
    return launched(dsa::launch_mla_decode(ls, (const uint16_t *)q, kv_cache, block_tables,
                                           seq_lens, sel, kv_scale, sm_scale, (uint16_t *)out,
                                           (char *)ws, wl, (hipStream_t)stream),
                    "mla_decode");
}

} // extern "C"

namespace {

// The whole step. ev: null, or 10 events bound in start/stop pairs to the
// index, filter, finish, attention and merge kernels.
int decode_k_impl(const dsa_shape *shape, const void *q_idx, const float *w, const void *k_normed,
                  const void *q, const uint8_t *kv_cache, const int32_t *block_tables,
                  const int32_t *seq_lens, float kv_scale, float sm_scale, float *scores,
                  int32_t *sel, void *out, void *ws, size_t ws_bytes, void *stream,
                  hipEvent_t const *ev)
{
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(q_idx, "q_idx")) || (rc = check_ptr(w, "w")) ||
        (rc = check_ptr(k_normed, "k_normed")) || (rc = check_ptr(q, "q")) ||
        (rc = check_ptr(kv_cache, "kv_cache")) || (rc = check_ptr(block_tables, "block_tables")) ||
        (rc = check_ptr(seq_lens, "seq_lens")) || (rc = check_ptr(scores, "scores")) ||
        (rc = check_ptr(sel, "sel")) || (rc = check_ptr(out, "out")))
        return rc;
    if (!(kv_scale > 0.0f) || !(sm_scale > 0.0f) || kv_scale == __builtin_huge_valf() ||
        sm_scale == __builtin_huge_valf())
        return fail(DSA_EINVAL, "kv_scale and sm_scale must be positive and finite");
    const dsa::Workspace wl = dsa::workspace_layout(ls);
    if ((rc = check_ws(ws, ws_bytes, wl)) != DSA_OK)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    char *wsb = (char *)ws;
    auto timer = [&](int stage) {
        dsa::KTimer t;
        if (ev != nullptr) {
            t.start = ev[2 * stage];
            t.stop = ev[2 * stage + 1];
        }
        return t;
    };
    // the group maxima only feed the threshold filter of long rows
    const bool gm = !dsa::select_direct(ls);
    if ((rc = launched(dsa::launch_index_scores(ls, (const uint16_t *)q_idx, w,
                                                (const uint16_t *)k_normed, seq_lens, scores,
                                                gm ? (uint32_t *)(wsb + wl.gm4) : nullptr,
                                                gm ? (uint32_t *)(wsb + wl.gm32) : nullptr, st,
                                                timer(0)),
                       "index_scores")) ||
        (rc = launched(dsa::launch_select(ls, scores, seq_lens, sel, wsb, wl, true, st, timer(1),
                                          timer(2)),
                       "select")) ||
        (rc = launched(dsa::launch_mla_decode(ls, (const uint16_t *)q, kv_cache, block_tables,
                                              seq_lens, sel, kv_scale, sm_scale, (uint16_t *)out,
                                              wsb, wl, st, timer(3), timer(4)),
                       "mla_decode")))
        return rc;
    return DSA_OK;
}

} // namespace

extern "C" {

int dsa_decode_k(const dsa_shape *shape, const void *q_idx, const float *w, const void *k_normed,
                 const void *q, const uint8_t *kv_cache, const int32_t *block_tables,
                 const int32_t *seq_lens, float kv_scale, float sm_scale, float *scores,
                 int32_t *sel, void *out, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    return decode_k_impl(shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens, kv_scale,
                         sm_scale, scores, sel, out, ws, ws_bytes, stream, nullptr);
}

int dsa_decode_k_timed(const dsa_shape *shape, const void *q_idx, const float *w,
                       const void *k_normed, const void *q, const uint8_t *kv_cache,
                       const int32_t *block_tables, const int32_t *seq_lens, float kv_scale,
                       float sm_scale, float *scores, int32_t *sel, void *out, void *ws,
                       size_t ws_bytes, void *stream, void *const *events)
{
    g_err[0] = 0;
    if (events == nullptr)
        return fail(DSA_EINVAL, "events is NULL");
    for (int i = 0; i < 10; i++)
        if (events[i] == nullptr)
            return fail(DSA_EINVAL, "events[%d] is NULL", i);
    return decode_k_impl(shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens, kv_scale,
                         sm_scale, scores, sel, out, ws, ws_bytes, stream,
                         (hipEvent_t const *)events);
}

int dsa_decode_k_noalloc(const dsa_shape *shape, const void *q_idx, const float *w,
                         const void *k_normed, const void *q, const uint8_t *kv_cache,
                         const int32_t *block_tables, const int32_t *seq_lens, float kv_scale,
                         float sm_scale, float *scores, int32_t *sel, void *out, void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    const size_t need = dsa::workspace_layout(ls).total;
    if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
        return fail(DSA_EWORKSPACE,
                    "this shape needs %zu bytes of workspace, above the %zu-byte scratch array of "
                    "dsa_decode_k_noalloc (use dsa_decode_k with a caller workspace)",
                    need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((rc = scratch_of_current_device(&ws)) != DSA_OK)
        return rc;
    // every part of the workspace is written before it is read within a call,
    // so the contents a previous call left need no clearing
    return dsa_decode_k(shape, q_idx, w, k_normed, q, kv_cache, block_tables, seq_lens, kv_scale,
                        sm_scale, scores, sel, out, ws, (size_t)DSA_NOALLOC_SCRATCH_BYTES, stream);
}

int dsa_cache_write(const dsa_shape *shape, const void *kv_a, const void *latent_w,
                    const void *k_proj, const void *k_w, const void *k_b,
                    const int32_t *seq_lens, const int32_t *block_tables, float eps,
                    float kv_scale, uint8_t *kv_cache, void *k_normed, uint8_t *valid,
                    void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if ((rc = check_ptr(kv_a, "kv_a")) || (rc = check_ptr(latent_w, "latent_w")) ||
        (rc = check_ptr(k_proj, "k_proj")) || (rc = check_ptr(k_w, "k_w")) ||
        (rc = check_ptr(k_b, "k_b")) || (rc = check_ptr(seq_lens, "seq_lens")) ||
        (rc = check_ptr(block_tables, "block_tables")) || (rc = check_ptr(kv_cache, "kv_cache")) ||
        (rc = check_ptr(k_normed, "k_normed")))
        return rc;
    if (!(eps >= 0.0f) || eps == __builtin_huge_valf())
        return fail(DSA_EINVAL, "eps must be finite and non-negative");
    if (!(kv_scale > 0.0f) || kv_scale == __builtin_huge_valf())
        return fail(DSA_EINVAL, "kv_scale must be positive and finite");
    return launched(dsa::launch_cache_write(ls, (const uint16_t *)kv_a, (const uint16_t *)latent_w,
                                            (const uint16_t *)k_proj, (const uint16_t *)k_w,
                                            (const uint16_t *)k_b, seq_lens, block_tables, eps,
                                            kv_scale, kv_cache, (uint16_t *)k_normed, valid,
                                            (hipStream_t)stream),
                    "cache_write");
}

int dsa_check_metadata(const dsa_shape *shape, const int32_t *seq_lens,
                       const int32_t *block_tables, const int32_t *sel, int where, void *stream)
{
    g_err[0] = 0;
    dsa::LaunchShape ls;
    int rc;
    if ((rc = check_shape(shape, &ls)) != DSA_OK)
        return rc;
    if (!seq_lens || !block_tables)
        return fail(DSA_EINVAL, "seq_lens and block_tables must not be NULL");
    if (where != DSA_META_DEVICE && where != DSA_META_HOST)
        return fail(DSA_EINVAL, "where %d is neither DSA_META_DEVICE nor DSA_META_HOST", where);
    const int R = ls.num_rows, S = ls.num_seqs, K = ls.rows_per_seq;
    const size_t n_bt = (size_t)S * ls.max_blocks;
    const size_t n_sel = sel ? (size_t)R * ls.top_k : 0;
    std::vector<int32_t> h_len, h_bt, h_sel;
    const int32_t *len = seq_lens, *bt = block_tables, *sl = sel;
    if (where == DSA_META_DEVICE) {
        hipStream_t st = (hipStream_t)stream;
        h_len.resize(R);
        h_bt.resize(n_bt);
        h_sel.resize(n_sel);
        if (hipMemcpyAsync(h_len.data(), seq_lens, R * sizeof(int32_t), hipMemcpyDeviceToHost,
                           st) != hipSuccess ||
            hipMemcpyAsync(h_bt.data(), block_tables, n_bt * sizeof(int32_t),
                           hipMemcpyDeviceToHost, st) != hipSuccess ||
            (sel && hipMemcpyAsync(h_sel.data(), sel, n_sel * sizeof(int32_t),
                                   hipMemcpyDeviceToHost, st) != hipSuccess) ||
            hipStreamSynchronize(st) != hipSuccess)
            return fail(DSA_ELAUNCH, "copying the metadata to the host failed: %s",
                        hipGetErrorString(hipGetLastError()));
        len = h_len.data();
        bt = h_bt.data();
        sl = sel ? h_sel.data() : nullptr;
    }
    long long bad = 0;
    char first[256] = "";
    auto note = [&](const char *fmt, auto... args) {
        if (bad++ == 0)
            snprintf(first, sizeof first, fmt, args...);
    };
    for (int r = 0; r < R; r++)
        if (len[r] < 0 || len[r] > ls.max_len)
            note("seq_lens[%d] = %d outside [0, max_len = %d]", r, len[r], ls.max_len);
    for (int s = 0; s < S; s++) {
        int lmax = 0;
        for (int j = 0; j < K; j++)
            lmax = std::max(lmax, std::min(std::max(len[s * K + j], 0), ls.max_len));
        const int nb = (lmax + ls.page_size - 1) / ls.page_size; // <= max_blocks
        for (int b = 0; b < nb; b++) {
            const int32_t p = bt[(size_t)s * ls.max_blocks + b];
            if (p < 0 || p >= ls.num_pages)
                note("block_tables[%d][%d] = %d outside [0, num_pages = %d] (sequence %d reaches "
                     "%d blocks)", s, b, p, ls.num_pages, s, nb);
        }
    }
    if (sl) {
        std::vector<int32_t> ids;
        for (int r = 0; r < R; r++) {
            const int L = std::min(std::max(len[r], 0), ls.max_len);
            const int n = std::min(ls.top_k, L);
            const int32_t *row = sl + (size_t)r * ls.top_k;
            ids.assign(row, row + n);
            for (int j = 0; j < n; j++)
                if (row[j] < 0 || row[j] >= L)
                    note("sel[%d][%d] = %d outside [0, L_r = %d)", r, j, row[j], L);
            std::sort(ids.begin(), ids.end());
            for (int j = 1; j < n; j++)
                if (ids[j] == ids[j - 1])
                    note("sel[%d] holds id %d more than once", r, ids[j]);
            for (int j = n; j < ls.top_k; j++)
                if (row[j] != -1)
                    note("sel[%d][%d] = %d past n_r = %d (padding must be -1)", r, j, row[j], n);
        }
    }
    if (bad)
        return fail(DSA_EMETADATA, "%lld out-of-contract value%s; first: %s", bad,
                    bad == 1 ? "" : "s", first);
    return DSA_OK;
}

} // extern "C"
