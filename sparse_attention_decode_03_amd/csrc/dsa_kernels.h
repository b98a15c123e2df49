// dsa_kernels.h -- host-side launchers of the gfx950 kernels (internal to
// libdsa; the public interface is include/dsa.h).
#pragma once

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

// Bins of the first selection histogram (top 11 bits of the score key).
constexpr int kHistBins = 2048;
constexpr int kHistShift = 21;

// Selection geometry: rows are cut into chunks of kSelChunk tokens.
constexpr int kSelChunk = 4096;
// Attention geometry: a row's selection is cut into chunks of kAttChunk
// slots; a workgroup covers kAttHeads heads of one chunk.
constexpr int kAttChunk = 256;
constexpr int kAttHeads = 64;

inline int sel_chunks(const LaunchShape &ls) { return (ls.max_len + kSelChunk - 1) / kSelChunk; }
inline int att_chunks(const LaunchShape &ls)
{
    const int n = ls.top_k < ls.max_len ? ls.top_k : ls.max_len;
    return (n + kAttChunk - 1) / kAttChunk;
}
inline int att_head_groups(const LaunchShape &ls) { return (ls.num_heads + kAttHeads - 1) / kAttHeads; }

// Per-row selection state in the workspace.
struct SelRow {
    uint32_t ticket;     // chunk workgroups of this row that have finished
    uint32_t thr_key;    // exact threshold key
    int32_t idx_cut;     // largest selected index among keys equal to thr_key
    uint32_t pad[5];
};

// Workspace carve-up (byte offsets, 256-aligned).
struct Workspace {
    size_t hist, selrow, clear_bytes; // [0, clear_bytes) is zeroed per call
    size_t n_gt, n_cand, offsets, cand;
    size_t part_o, part_ml;
    size_t total;
};
Workspace workspace_layout(const LaunchShape &ls);

int launch_clear(void *ws, size_t bytes, hipStream_t stream);
int launch_index_scores(const LaunchShape &ls, const uint16_t *q_idx, const float *w,
                        const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                        uint32_t *hist, hipStream_t stream);
int launch_score_hist(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                      uint32_t *hist, hipStream_t stream);
int launch_select(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                  int32_t *sel, char *ws, const Workspace &wl, hipStream_t stream);
int launch_mla_decode(const LaunchShape &ls, const uint16_t *q, const uint8_t *kv_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, const int32_t *sel,
                      float kv_scale, float sm_scale, uint16_t *out, char *ws,
                      const Workspace &wl, hipStream_t stream);

} // namespace dsa
