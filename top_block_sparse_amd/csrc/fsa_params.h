// fsa_params.h -- kernel parameter blocks and launcher declarations of libfsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fsa {

// Selected-attention prefill (sel_attn_fwd.hip).
struct SelFwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* blk_idx;
    const int32_t* cu_q;
    const int32_t* cu_k;
    uint16_t* out;
    float* lse;
    float* part_o;      // [num_splits][total_q*Hq][D]   (num_splits > 1)
    float* part_lse;    // [num_splits][total_q*Hq]
    int64_t total_q;
    int64_t total_k;
    int batch, Hq, Hkv, G, topk, num_splits;
    int wl, wr;         // key window of row i: [i + off - wl, i + off + wr], -1 = unlimited
    int dense;          // 1: every key of the window (no block lists; blk_idx unused)
    int T;              // query tokens per tile (<= 64)
    int mtiles;         // ceil(T*G/16) 16-row MFMA tiles per tile
    int tiles_per_seq;
    int n_wg;
    int head_major;     // 1: all XCDs on one (sequence, kv head) unit at a time
    int ring;           // LDS ring slots of K/V blocks (3 or 4)
    int spin_limit;     // polls before a ring wait gives up
    float scale_log2;   // softmax_scale * log2(e)
};

// Selected-attention prefill, block-centric schedule (sel_attn_fwd_bc.hip).
struct SelFwdBcParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* blk_idx;
    const int32_t* cu_q;
    const int32_t* cu_k;
    uint16_t* out;
    float* lse;
    // workspace
    int32_t* counts;             // [units][nb_max + 1]: entries per block, then offsets
    int32_t* cursor;             // [units][nb_max]: fill cursors
    unsigned long long* masks;   // [total_q][Hkv]: list slots that count
    int32_t* ents;               // [total_q * Hkv * topk]: token << 6 | slot, grouped by block
    int32_t* pos;                // [total_q][Hkv][topk]: where the fill pass put each entry
    int2* tasks;                 // [max_tasks]: (unit * nb_max + block, first tile)
    uint32_t* ctr;               // [16]: [0] tasks written, [8 + x] next task of segment x
    float* part_ml;              // [entry][G][2]: log2-domain max and sum, in ents order
    uint16_t* part_o;            // [entry][G][D] bf16 partials (not divided by the sum)
    int64_t total_q, total_k;
    int batch, Hq, Hkv, G, topk, causal, nb_max;
    int tpt;                     // tokens per 16-row tile
    int nchunk_q;                // index workgroups per (sequence, kv head)
    int max_tasks;
    int n_wg;                    // main-kernel workgroups (persistent)
    float scale_log2;
};

// Top-k paged decode (topk_decode.hip).
struct DecodeParams {
    const uint16_t* q;
    const void* kc;         // bf16, or FP8 E4M3 bytes when kv_fp8
    const void* vc;
    const float* k_descale; // [batch*Hkv] or null (kv_fp8 only)
    const float* v_descale;
    const int32_t* tok_idx;
    const int32_t* block_table;
    const int32_t* cache_seqlens;
    uint16_t* out;          // [batch*Hq][D] bf16 (splits == 1)
    float* lse;             // optional [batch*Hq] (splits == 1)
    float* part_o;          // workspace: [splits][batch*Hq][D] (splits > 1)
    float* part_lse;        // workspace: [splits][batch*Hq]
    int batch, Hq, Hkv, G, page_size, max_pages, num_pages, topk, splits;
    int ts;                 // hash table slots (> topk)
    int kv_fp8;
    float scale_log2;
};

// Block-index producer (block_select.hip).
// Row stride, in floats, of its importance table [T][blocks] in LDS: rows of
// more than 16 blocks are padded to 16 (mod 64) floats, so that 16-lane groups
// that read or add to four different rows fall in four different bank ranges.
inline __host__ __device__ int select_row_stride(int nb) { return nb <= 16 ? nb : nb + ((16 - nb) & 63); }

struct BlockSelectParams {
    const uint16_t* q;
    const uint16_t* k;
    const int32_t* cu_q;
    const int32_t* cu_k;
    uint16_t* cmp;          // workspace: compressed keys [batch][ncmp_max][Hkv][D] bf16
    int32_t* blk_idx;       // [total_q][Hkv][topk]
    int64_t total_q, total_k;
    int batch, Hq, Hkv, G, topk, init, local;
    int ncmp_max;           // windows of the longest sequence
    int nb_max;             // blocks of the longest sequence
    int T, mtiles, tiles_per_seq;
    float scale_log2;
};

// Selected-attention backward (sel_attn_bwd.hip).
struct SelBwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;        // [Hq][total_q], natural log (the forward's)
    const int32_t* blk_idx;
    const int32_t* cu_q;
    const int32_t* cu_k;
    uint16_t* dq;            // [total_q][Hq][D]
    uint16_t* dk;            // [total_k][Hkv][D]
    uint16_t* dv;
    float* dvec;             // workspace [Hq][total_q]: rowsum(dO * O)
    int32_t* counts;         // workspace [batch*Hkv][nb_max + 1]: counts, then offsets
    int32_t* cursor;         // workspace [batch*Hkv][nb_max]
    int32_t* toks;           // workspace [total_q * Hkv * topk]: token lists per block
    float* kv_acc;           // workspace [total_k][Hkv][2][D] fp32: dK, dV of split blocks
    int64_t total_q, total_k;
    int batch, Hq, Hkv, G, topk, causal, nb_max;
    int nparts, part_steps;  // a block's 32-row steps go to <= nparts workgroups of part_steps
    int T, mtiles, tiles_per_seq;   // dq tiling
    int ring;                       // dq LDS ring slots of K/V blocks (2..4)
    int spin_limit;                 // polls before a ring wait gives up
    int nchunk_q;                   // index workgroups per (sequence, kv head)
    float scale, scale_log2;
};

// Logsumexp merge of split partials (lse_merge.hip).
struct MergeParams {
    const float* part_o;     // [nparts][nrows][D]
    const float* part_lse;   // [nparts][nrows]
    uint16_t* out;           // [nrows][D] bf16
    float* lse;              // optional
    int64_t nrows;
    int nparts;
    int lse_mode;            // 0: lse[(row % Hq) * ntok + row / Hq]; 1: lse[row]
    int Hq;
    int64_t ntok;
    const int32_t* ntok_live;   // optional: rows of tokens >= *ntok_live are left untouched
};

// Polls a ring wait makes before it gives up (normal waits take ~1e3).
constexpr int kDefaultSpinLimit = 1 << 22;
// Device counters of ring waits that gave up, per kernel file (read and
// optionally cleared; synchronous).
hipError_t sel_attn_fwd_wait_timeouts(unsigned int* n, bool reset);
hipError_t sel_attn_bwd_wait_timeouts(unsigned int* n, bool reset);

template <int D>
hipError_t launch_sel_attn_fwd(const SelFwdParams& p, hipStream_t stream);
hipError_t launch_sel_attn_fwd_bc(const SelFwdBcParams& p, int D, hipStream_t stream);
constexpr int kBcTileTasks = 64;      // 16-row tiles per block-centric task
constexpr int kBcIndexChunk = 256;    // tokens per index workgroup
constexpr int kBcWgPerCu = 2;         // resident main-kernel workgroups per CU
size_t sel_attn_fwd_lds_bytes(int D, int T, int topk, int ring);
int sel_attn_fwd_ring(int D, int T, int topk);   // ring slots that fit in LDS
int sel_attn_fwd_rows_per_tile();   // query rows (T*G) one workgroup covers
hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t stream);
int decode_waves_per_workgroup(int G);
size_t decode_lds_bytes(int D, int G, int ts, int topk);
int decode_table_slots(int D, int G, int topk);
hipError_t launch_lse_merge(const MergeParams& p, int D, hipStream_t stream);
hipError_t launch_sel_attn_bwd(const SelBwdParams& p, int D, hipStream_t stream);
hipError_t launch_block_select(const BlockSelectParams& p, int D, hipStream_t stream);
size_t block_select_lds_bytes(int T, int nb_max, int D);
int sel_attn_bwd_rows_per_tile();   // query rows (T*G) one dq workgroup covers
int sel_attn_bwd_index_chunk();     // tokens one index workgroup covers
size_t sel_attn_bwd_dq_lds_bytes(int D, int T, int topk, int ring);
int sel_attn_bwd_dq_ring(int D, int T, int topk);   // ring slots that fit in LDS (0: none)

}  // namespace fsa
