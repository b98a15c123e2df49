// dsa_kernels.h -- host-side launchers of the gfx950 kernels (internal to
// libdsa; the public interface is include/dsa.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Validated copy of the public dsa_shape with derived sizes.
struct LaunchShape {
    int num_seqs, rows_per_seq, num_rows;
    int num_heads, latent_dim;
    int index_heads, index_dim;
    int top_k, page_size, max_len, k_capacity, max_blocks, num_pages;
};

// Selection: radix digits of up to 11 bits (2048 bins); the filter pass
// cuts each row into slices of kSelSlice tokens.
constexpr int kHistBins = 2048;
constexpr int kSelSlice = 4096;
inline int sel_slices(const LaunchShape &ls) { return (ls.max_len + kSelSlice - 1) / kSelSlice; }

// Attention geometry: a row's selection is cut into chunks of kAttChunk
// slots; a workgroup covers up to kAttHeads heads of one chunk. 256 slots
// (8 steps of 32 tokens) per chunk: measured on gfx950 against 128, the
// longer pipeline per workgroup and the halved partial traffic take the
// K-token verify step from 122 to 109 us, with the long-context step
// unchanged within noise (it then runs 16-head workgroups).
constexpr int kAttChunk = 256;
constexpr int kAttHeads = 64;

// Row stride of the scores buffer: max_len rounded up to 64 floats, so every
// row starts 256-byte aligned.
inline int score_stride(const LaunchShape &ls) { return (ls.max_len + 63) / 64 * 64; }

// Index-score pass geometry: 256-token tiles, 128 for units of two or four
// rows and for calls with few tiles (the balance of tiles over workgroups is
// computed on the device from the lengths).
constexpr int kIdxTile = 256;
// A last tile this short does not count as a tile of work in the split.
constexpr int kIdxLightTail = 32;
// Rows per sequence the boundary accepts (K of a verify or row group).
constexpr int kMaxRowsPerSeq = 16;

inline int att_chunks(const LaunchShape &ls)
{
    const int n = ls.top_k < ls.max_len ? ls.top_k : ls.max_len;
    return (n + kAttChunk - 1) / kAttChunk;
}
inline int att_head_groups(const LaunchShape &ls) { return (ls.num_heads + kAttHeads - 1) / kAttHeads; }

// Workspace carve-up (byte offsets, 256-aligned). Nothing needs zeroing:
// every part is written before it is read within a call.
struct Workspace {
    size_t cand;    // [R][score_stride] (key, index) selection candidates
    size_t bitmap;  // [R][score_stride / 32] selection bitmaps of long rows
    size_t cnt;     // [R][sel_slices] candidates per slice
    size_t gm4;     // [R][score_stride / 4] max key of each 4-token group
    size_t gm32;    // [R][score_stride / 32] max key of each 32-token group
    size_t part_o, part_ml; // per-chunk attention partials: bf16 O, fp32 (m, l)
    size_t total;
};
Workspace workspace_layout(const LaunchShape &ls);

// Start and stop events bound to one kernel's dispatch: hipExtLaunchKernel
// stamps them with that dispatch's own begin and end, so their span is the
// kernel's run alone. Both null: an untimed launch.
struct KTimer {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// gm4 / gm32 null: scores only. Otherwise the pass also writes the group
// maxima the selection threshold is taken from.
int launch_index_scores(const LaunchShape &ls, const uint16_t *q_idx, const float *w,
                        const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                        uint32_t *gm4, uint32_t *gm32, hipStream_t stream, KTimer t = {});
// Rows of at most kSelDirectMax tokens (by the shape's max_len) are
// selected by one kernel that holds the whole row (no group maxima needed);
// longer ones by the threshold filter and the finish. The one kernel costs
// more per row as rows grow (8.6 us at 8 tokens a thread, 13.4 at 16, 18.9
// at 24, 21.8 at 32), the two kernels about 16-17 us whatever the length,
// but the one kernel also spares the index pass its group maxima (2.6 us at
// 64 rows x 16.4k) and a kernel boundary: it wins up to 24 tokens a thread.
constexpr int kSelDirectMax = 24576;
inline bool select_direct(const LaunchShape &ls) { return ls.max_len <= kSelDirectMax; }
// have_group_max: the group maxima in the workspace were written by the
// index pass of the same call; otherwise the selection computes them first
// (neither matters with select_direct).
// t_filter / t_finish time the filter and the finish kernels (with
// select_direct: the finish's pair times the one kernel, the filter's spans
// nothing).
int launch_select(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                  int32_t *sel, char *ws, const Workspace &wl, bool have_group_max,
                  hipStream_t stream, KTimer t_filter = {}, KTimer t_finish = {});
// Pooled selection of pool_scores [R][score_stride(ls_pool)] over per-row
// pool counts L_r / kp, expanded to token ids in sel [R][top_k * kp + kp - 1].
// ls_pool is the token shape with max_len = max(1, max_len / kp); pool counts
// and selected pools live in the workspace at the given offsets; any_pool
// false (max_len < kp) skips the selection (every row keeps its tail only).
// pool_valid [S][score_stride(ls_pool)] (may be null): a pool marked 0 is no
// candidate (its score goes to -inf in the `masked` region before the
// selection, and the expansion drops it if it was still taken).
int launch_select_pooled(const LaunchShape &ls_pool, int max_len, int kp, const float *pool_scores,
                         const uint8_t *pool_valid, const int32_t *seq_lens, int32_t *sel, char *ws,
                         const Workspace &wl, size_t pool_lens_off, size_t sel_pools_off,
                         size_t masked_off, bool any_pool, hipStream_t stream);
int launch_cache_write(const LaunchShape &ls, const uint16_t *kv_a, const uint16_t *latent_w,
                       const uint16_t *k_proj, const uint16_t *k_w, const uint16_t *k_b,
                       const int32_t *seq_lens, const int32_t *block_tables, float eps,
                       float kv_scale, uint8_t *kv_cache, uint16_t *k_normed, uint8_t *valid,
                       hipStream_t stream);
// t_att / t_merge time the attention and the merge kernels; with a single
// chunk there is no merge and t_merge's events, if any, are recorded right
// after the attention (a span of about zero).
int launch_mla_decode(const LaunchShape &ls, const uint16_t *q, const uint8_t *kv_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                      float kv_scale, float sm_scale, uint16_t *out, char *ws,
                      const Workspace &wl, hipStream_t stream, KTimer t_att = {},
                      KTimer t_merge = {});

} // namespace dsa
