// fsa_api.hip -- host side of libfsa: argument checks, planning, launches.
//
// The entry points are declared (with their contracts) in include/fsa.h.
// Nothing here allocates, frees or synchronises device memory; every check
// runs before the first launch so a rejected call leaves the device
// untouched.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/fsa.h"
#include "fsa_common.h"
#include "fsa_params.h"

namespace {

constexpr int kMaxTopkPrefill = 64;
constexpr int kMaxGroupPrefill = 224;   // one tile covers at most 14 m-tiles of 16 rows
constexpr int kMaxSplitsPrefill = 16;
constexpr int kMaxGroupBackward = 32;   // 32 query rows per dK/dV step hold one token at least
constexpr int kMaxTopkDecode = 8192;
constexpr int kMaxGroupDecode = 16;
constexpr int kMaxSplitsDecode = 64;
constexpr size_t kAlign = 256;

// Polls a ring wait makes before it gives up (fsa_set_wait_poll_limit).
std::atomic<int> g_spin_limit{fsa::kDefaultSpinLimit};

// Every launch of one call is checked on the host before the first one is
// enqueued: at most kMaxGroups workgroups (of up to 1024 work-items, so the
// dispatch size stays within 32 bits).
constexpr long long kMaxGroups = 1ll << 22;
bool groups_ok(long long g) { return g >= 0 && g <= kMaxGroups; }

// No sequence is longer than the rows it lives in: the caller's maximum
// lengths are capped by the totals (which keeps every derived grid and
// workspace size bounded by the tensors themselves).
int32_t cap_len(int32_t max_len, int64_t total) {
    return (int64_t)max_len > total ? (int32_t)total : max_len;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Prefill tiling: T tokens per workgroup so that T*G query rows fill at most
// 16 MFMA m-tiles, and at most 64 tokens (one bit each in the block masks).
struct PrefillPlan {
    int T, mtiles, tiles_per_seq, splits, n_wg, head_major;
};

// Tile order of the query-centric kernel.  When one (sequence, kv head) unit's
// K and V exceed kHeadMajorBytes they cannot stay in one XCD's 4 MiB L2, and
// the tiles of all units would compete for the 256 MiB Infinity Cache at once;
// then every XCD works through the same unit at the same time, each on every
// eighth tile (measured at 131072 tokens x 4 kv heads, d 128: 27.9 ms against
// 32.8 ms).  Smaller units keep one XCD each.
constexpr long long kHeadMajorBytes = 8ll << 20;

void set_tile_order(PrefillPlan& pl, int32_t batch, int32_t Hkv, int32_t max_seqlen_k, int32_t D) {
    if ((long long)max_seqlen_k * D * 2 * 2 <= kHeadMajorBytes) return;
    const long long n = (long long)batch * Hkv * pl.splits * ((pl.tiles_per_seq + 7) / 8) * 8;
    if (!groups_ok(n)) return;
    pl.head_major = 1;
    pl.n_wg = (int)n;
}

// num_splits: 0 automatic, n >= 1 query-centric with n splits, -1 block-centric
// (selected attention only; checked by the caller against the group size).
fsa_status_t check_prefill_shape(int32_t batch, int32_t max_seqlen_q, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t bs, int32_t topk, int32_t num_splits) {
    if (batch < 0 || max_seqlen_q < 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 || num_splits < -1)
        return FSA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FSA_ERROR_INVALID_VALUE;
    if (D != 64 && D != 128) return FSA_ERROR_NOT_SUPPORTED;
    if (bs != fsa::kBlockKeys) return FSA_ERROR_NOT_SUPPORTED;
    if (topk > kMaxTopkPrefill) return FSA_ERROR_NOT_SUPPORTED;
    if (Hq / Hkv > kMaxGroupPrefill) return FSA_ERROR_NOT_SUPPORTED;
    if (num_splits > kMaxSplitsPrefill) return FSA_ERROR_NOT_SUPPORTED;
    return FSA_SUCCESS;
}

PrefillPlan plan_prefill(int32_t batch, int32_t max_seqlen_q, int32_t Hq, int32_t Hkv,
                         int32_t num_splits) {
    PrefillPlan pl{};
    const int G = Hq / Hkv;
    int T = fsa::sel_attn_fwd_rows_per_tile() / G;
    if (T > 64) T = 64;
    if (T < 1) T = 1;
    pl.T = T;
    pl.mtiles = (T * G + 15) / 16;
    pl.tiles_per_seq = (int)(((long long)max_seqlen_q + T - 1) / T);
    const long long base = (long long)batch * pl.tiles_per_seq * Hkv;
    int s = num_splits;
    if (s == 0) {
        // enough workgroups to cover 256 CUs a few times over
        s = 1;
        if (base > 0 && base < 1024) {
            s = (int)((1024 + base - 1) / base);
            if (s > 8) s = 8;
        }
    }
    pl.splits = s;
    pl.n_wg = groups_ok(base * s) ? (int)(base * s) : -1;      // -1: too many workgroups
    pl.head_major = 0;
    return pl;
}

// Enough workgroups to give every CU one (each splits list entries among
// its waves; a split list repeats the set computation in every part), with
// at least 32 entries per wave.
int decode_auto_splits(int32_t batch, int32_t Hq, int32_t Hkv, int32_t topk) {
    const long long units = (long long)batch * Hkv;
    if (units <= 0 || Hkv <= 0) return 1;
    const int waves = fsa::decode_waves_per_workgroup(Hq / Hkv);
    long long s = (256 * 8 + units * waves - 1) / (units * waves);
    const long long cap = topk / (waves * 32) > 1 ? topk / (waves * 32) : 1;
    if (s > cap) s = cap;
    if (s > kMaxSplitsDecode) s = kMaxSplitsDecode;
    if (s < 1) s = 1;
    return (int)s;
}

fsa_status_t check_decode_shape(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D, int32_t topk,
                                int32_t num_splits) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 || num_splits < 0)
        return FSA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FSA_ERROR_INVALID_VALUE;
    if (D != 64 && D != 128) return FSA_ERROR_NOT_SUPPORTED;
    if (topk > kMaxTopkDecode) return FSA_ERROR_NOT_SUPPORTED;
    if (Hq / Hkv > kMaxGroupDecode) return FSA_ERROR_NOT_SUPPORTED;
    if (num_splits > kMaxSplitsDecode) return FSA_ERROR_NOT_SUPPORTED;
    return FSA_SUCCESS;
}

// Decode workspace: split partials only (none when the lists are not split).
struct DecodeLayout {
    size_t part_o, part_lse, total;
    int splits;
};

DecodeLayout decode_layout(int32_t batch, int32_t Hq, int32_t Hkv, int32_t D, int32_t topk,
                           int32_t num_splits) {
    DecodeLayout l{};
    l.splits = num_splits == 0 ? decode_auto_splits(batch, Hq, Hkv, topk) : num_splits;
    if (l.splits <= 1) return l;
    size_t off = 0;
    l.part_o = off;
    off = align_up(off + (size_t)l.splits * batch * Hq * D * 4);
    l.part_lse = off;
    off = align_up(off + (size_t)l.splits * batch * Hq * 4);
    l.total = off;
    return l;
}

float resolve_scale(float s, int D) { return s > 0.f ? s : 1.0f / std::sqrt((float)D); }

// Block-index producer: the importance table [T][blocks] (fp32) of one tile
// lives in LDS; T tokens times G heads fill at most 8 m-tiles of 16 rows.
constexpr int kSelectCmpSize = 32, kSelectCmpStride = 16;
constexpr int kMaxTopkSelect = 64;
constexpr int kMaxGroupSelect = 128;
constexpr size_t kSelectLdsBudget = 64 * 1024;

struct SelectPlan {
    int T, mtiles, tiles_per_seq, ncmp_max, nb_max;
};

fsa_status_t check_select(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t ks, int32_t stride, int32_t bs,
                          int32_t topk, int32_t init, int32_t local) {
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 ||
        init < 0 || local < 0 || ks <= 0 || stride <= 0 || bs <= 0)
        return FSA_ERROR_INVALID_VALUE;
    if (Hq % Hkv != 0) return FSA_ERROR_INVALID_VALUE;
    if (D != 64 && D != 128) return FSA_ERROR_NOT_SUPPORTED;
    if (ks != kSelectCmpSize || stride != kSelectCmpStride || bs != fsa::kBlockKeys)
        return FSA_ERROR_NOT_SUPPORTED;
    if (topk > kMaxTopkSelect || Hq / Hkv > kMaxGroupSelect) return FSA_ERROR_NOT_SUPPORTED;
    return FSA_SUCCESS;
}

SelectPlan plan_select(int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv) {
    SelectPlan pl{};
    const int G = Hq / Hkv;
    pl.nb_max = (int)(((long long)max_seqlen_k + fsa::kBlockKeys - 1) / fsa::kBlockKeys);
    if (pl.nb_max < 1) pl.nb_max = 1;
    pl.ncmp_max = max_seqlen_k >= kSelectCmpSize ? (max_seqlen_k - kSelectCmpSize) / kSelectCmpStride + 1 : 0;
    int T = 128 / G;                            // 8 m-tiles of 16 rows
    // (the table's rows are padded in LDS -- select_row_stride -- by at most 63
    // floats; the budget is on the unpadded rows, so the padding never changes
    // which lengths fit, and the padded table stays under 64 KiB + T * 252 B)
    const int t_lds = (int)(kSelectLdsBudget / ((size_t)pl.nb_max * 4));
    T = T < t_lds ? T : t_lds;
    // rows over 512 windows run the two-pass kernel, whose 32 KiB of chunk
    // buffers sit beside the table: at most 40 KiB of table (unpadded) lets
    // two of its workgroups share a CU (2048 blocks: T = 5, 73.5 -> 63.7 ms
    // at 131072 tokens); the support rule above is unchanged
    if (pl.ncmp_max > 512 && T > 0) {
        int t2 = (int)(40 * 1024 / ((size_t)pl.nb_max * 4));
        t2 = t2 < 1 ? 1 : t2;
        T = T < t2 ? T : t2;
    }
    pl.T = T;                                   // 0: the table does not fit
    pl.mtiles = (T * G + 15) / 16;
    pl.tiles_per_seq = T > 0 ? (int)(((long long)max_seqlen_q + T - 1) / T) : 0;
    return pl;
}

}  // namespace

// ---- fsa_topk_decode_noalloc: the split partials of the decode (the only
// scratch its kernels use) go to this library-owned array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a stand-in for the symbol:
// its device address (per device) comes from hipGetSymbolAddress on the
// first call on that device and is the one ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = (size_t)FSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

static fsa_status_t noalloc_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FSA_ERROR_LAUNCH;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        // (racing first calls on one device obtain the same address)
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return FSA_ERROR_LAUNCH;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return FSA_SUCCESS;
}

static fsa_status_t decode_impl(const void* q, const void* k_cache, const void* v_cache,
                               bool kv_fp8, const float* k_descale, const float* v_descale,
                             const int32_t* tok_idx, const int32_t* block_table,
                             const int32_t* cache_seqlens, int32_t batch, int32_t num_heads_q,
                             int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
                             int32_t max_pages_per_seq, int32_t num_pages, int32_t topk,
                             float softmax_scale, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, void* stream) {
    fsa_status_t st = check_decode_shape(batch, num_heads_q, num_heads_kv, head_dim, topk,
                                         num_splits);
    if (st != FSA_SUCCESS) return st;
    if (page_size <= 0 || max_pages_per_seq < 0 || num_pages < 0) return FSA_ERROR_INVALID_VALUE;
    if ((int64_t)num_pages * page_size >= (int64_t)INT32_MAX) return FSA_ERROR_NOT_SUPPORTED;
    if (batch == 0) return FSA_SUCCESS;
    if (!q || !k_cache || !v_cache || !tok_idx || !block_table || !cache_seqlens || !out)
        return FSA_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return FSA_ERROR_INVALID_VALUE;
    const DecodeLayout lay = decode_layout(batch, num_heads_q, num_heads_kv, head_dim, topk,
                                           num_splits);
    if (!groups_ok((long long)batch * num_heads_kv * lay.splits) ||
        !groups_ok(((long long)batch * num_heads_q + 3) / 4))
        return FSA_ERROR_NOT_SUPPORTED;
    if (lay.total > 0 && (workspace == nullptr || workspace_bytes < lay.total ||
                          (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0))
        return FSA_ERROR_WORKSPACE;

    fsa::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.kc = k_cache;
    p.vc = v_cache;
    p.kv_fp8 = kv_fp8 ? 1 : 0;
    p.k_descale = k_descale;
    p.v_descale = v_descale;
    p.tok_idx = tok_idx;
    p.block_table = block_table;
    p.cache_seqlens = cache_seqlens;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    if (lay.splits > 1) {
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        p.part_o = reinterpret_cast<float*>(ws + lay.part_o);
        p.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
    }
    p.batch = batch;
    p.Hq = num_heads_q;
    p.Hkv = num_heads_kv;
    p.G = num_heads_q / num_heads_kv;
    p.page_size = page_size;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    p.topk = topk;
    p.splits = lay.splits;
    p.ts = fsa::decode_table_slots(head_dim, p.G, topk);
    p.scale_log2 = resolve_scale(softmax_scale, head_dim) * fsa::kLog2e;
    if (fsa::decode_lds_bytes(head_dim, p.G, p.ts, topk) > 160 * 1024)
        return FSA_ERROR_NOT_SUPPORTED;

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (fsa::launch_decode(p, head_dim, s) != hipSuccess) return FSA_ERROR_LAUNCH;
    if (lay.splits > 1) {
        fsa::MergeParams m{};
        m.part_o = p.part_o;
        m.part_lse = p.part_lse;
        m.out = p.out;
        m.lse = lse;
        m.nrows = (int64_t)batch * num_heads_q;
        m.nparts = lay.splits;
        m.lse_mode = 1;
        m.Hq = num_heads_q;
        m.ntok = batch;
        if (fsa::launch_lse_merge(m, head_dim, s) != hipSuccess) return FSA_ERROR_LAUNCH;
    }
    return FSA_SUCCESS;
}

size_t prefill_workspace(const PrefillPlan& pl, int64_t total_q, int32_t Hq, int32_t D) {
    if (pl.splits <= 1) return 0;
    const size_t rows = (size_t)total_q * Hq;
    return align_up((size_t)pl.splits * rows * D * 4) + align_up((size_t)pl.splits * rows * 4);
}

// Block-centric schedule (sel_attn_fwd_bc.hip): the automatic choice for
// selected attention with a GQA group of at most kMaxGroupBc, where a token's
// rows fill a small fraction of an MFMA tile (the FSA page keeps its loop swap
// for groups below 8 and falls back to the query-centric kernel above).
// Measured on MI355X: at G = 1 (varlen 65536 + 32768, topk 16) 1.31 ms against
// 8.8 ms query-centric; at G = 4 (2 x 8192, topk 16) 1.33 ms against 0.90 ms,
// where the bf16 partial round trip through HBM costs more than the padding
// it removes.
constexpr int kMaxGroupBc = 2;
constexpr int kMaxSeqBc = 1 << 25;      // token index within a sequence << 6 must fit int32

constexpr int kMaxGroupBcForced = 16;   // a 16-row MFMA tile holds at least one token
constexpr int32_t kSplitsBlockCentric = -1;

bool use_block_centric(int32_t G, int32_t num_splits, int32_t max_seqlen_q, int64_t total_q,
                       int32_t Hkv, int32_t topk) {
    if (max_seqlen_q >= kMaxSeqBc) return false;
    if (total_q * Hkv * topk > INT32_MAX) return false;      // entry positions are int32
    if (num_splits == kSplitsBlockCentric) return G <= kMaxGroupBcForced;
    return num_splits == 0 && G <= kMaxGroupBc;
}

struct BcLayout {
    size_t counts, cursor, masks, ents, pos, tasks, ctr, part_ml, part_o, total;
    int nb_max, tpt, max_tasks;
};

BcLayout bc_layout(int32_t batch, int64_t total_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                   int32_t D, int32_t topk) {
    BcLayout l{};
    const int G = Hq / Hkv;
    l.tpt = 16 / G;
    l.nb_max = (max_seqlen_k + fsa::kBlockKeys - 1) / fsa::kBlockKeys;
    if (l.nb_max < 1) l.nb_max = 1;
    const size_t units = (size_t)batch * Hkv;
    const size_t entries = (size_t)total_q * Hkv * topk;
    // each block's entries make at most n_b / (tpt * tiles per task) + 1 tasks
    const size_t mt = entries / ((size_t)l.tpt * fsa::kBcTileTasks) + units * l.nb_max + 1;
    l.max_tasks = mt > (size_t)INT32_MAX ? INT32_MAX : (int)mt;
    size_t off = 0;
    l.counts = off;
    off = align_up(off + units * (l.nb_max + 1) * 4);
    l.cursor = off;
    off = align_up(off + units * l.nb_max * 4);
    l.masks = off;
    off = align_up(off + (size_t)total_q * Hkv * 8);
    l.ents = off;
    off = align_up(off + entries * 4);
    l.pos = off;
    off = align_up(off + entries * 4);
    l.tasks = off;
    off = align_up(off + (size_t)l.max_tasks * 8);
    l.ctr = off;
    off = align_up(off + 16 * 4);
    // (+16 rows: a dummy partial row per tile row for lanes with no entry)
    l.part_ml = off;
    off = align_up(off + (entries * G + 16) * 8);
    l.part_o = off;
    off = align_up(off + (entries * G + 16) * D * 2);
    l.total = off;
    return l;
}

static fsa_status_t prefill_bc(const void* q, const void* k, const void* v, const int32_t* blk_idx,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int64_t total_q, int64_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads_q,
                               int32_t num_heads_kv, int32_t head_dim, int32_t topk,
                               float softmax_scale, bool causal,
                               void* workspace, size_t workspace_bytes, void* out, float* lse,
                               void* stream) {
    const BcLayout lay = bc_layout(batch, total_q, max_seqlen_k, num_heads_q, num_heads_kv,
                                   head_dim, topk);
    if (workspace == nullptr || workspace_bytes < lay.total ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return FSA_ERROR_WORKSPACE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return FSA_ERROR_LAUNCH;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    fsa::SelFwdBcParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.blk_idx = blk_idx;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.counts = reinterpret_cast<int32_t*>(ws + lay.counts);
    p.cursor = reinterpret_cast<int32_t*>(ws + lay.cursor);
    p.masks = reinterpret_cast<unsigned long long*>(ws + lay.masks);
    p.ents = reinterpret_cast<int32_t*>(ws + lay.ents);
    p.pos = reinterpret_cast<int32_t*>(ws + lay.pos);
    p.tasks = reinterpret_cast<int2*>(ws + lay.tasks);
    p.ctr = reinterpret_cast<uint32_t*>(ws + lay.ctr);
    p.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
    p.part_o = reinterpret_cast<uint16_t*>(ws + lay.part_o);
    p.total_q = total_q;
    p.total_k = total_k;
    p.batch = batch;
    p.Hq = num_heads_q;
    p.Hkv = num_heads_kv;
    p.G = num_heads_q / num_heads_kv;
    p.topk = topk;
    p.causal = causal ? 1 : 0;
    p.nb_max = lay.nb_max;
    p.tpt = lay.tpt;
    p.max_tasks = lay.max_tasks;
    p.nchunk_q = (int)(((long long)max_seqlen_q + fsa::kBcIndexChunk - 1) / fsa::kBcIndexChunk);
    const int rows_per_merge_wg = 256 / (head_dim / 8);
    if (!groups_ok((long long)batch * num_heads_kv * p.nchunk_q) ||
        !groups_ok(((long long)total_q * num_heads_q + rows_per_merge_wg - 1) / rows_per_merge_wg))
        return FSA_ERROR_NOT_SUPPORTED;
    const long long nwg = (long long)cus * fsa::kBcWgPerCu;
    p.n_wg = (int)(nwg < lay.max_tasks ? nwg : lay.max_tasks);
    if (p.n_wg < 1) p.n_wg = 1;
    p.scale_log2 = resolve_scale(softmax_scale, head_dim) * fsa::kLog2e;
    (void)hipGetLastError();
    if (fsa::launch_sel_attn_fwd_bc(p, head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
        return FSA_ERROR_LAUNCH;
    return FSA_SUCCESS;
}

static fsa_status_t prefill_impl(const void* q, const void* k, const void* v,
                                 const int32_t* blk_idx, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t batch, int64_t total_q,
                                 int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                 int32_t block_size, int32_t topk, float softmax_scale,
                                 int32_t wl, int32_t wr, bool dense, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, void* out, float* lse,
                                 void* stream) {
    fsa_status_t st = check_prefill_shape(batch, max_seqlen_q, num_heads_q, num_heads_kv, head_dim,
                                          block_size, topk, num_splits);
    if (st != FSA_SUCCESS) return st;
    if (total_q < 0 || total_k < 0 || max_seqlen_k < 0) return FSA_ERROR_INVALID_VALUE;
    if (total_q > INT32_MAX || total_k > INT32_MAX) return FSA_ERROR_NOT_SUPPORTED;
    max_seqlen_q = cap_len(max_seqlen_q, total_q);
    max_seqlen_k = cap_len(max_seqlen_k, total_k);
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FSA_SUCCESS;   // nothing to do
    if (!q || !k || !v || (!dense && !blk_idx) || !cu_seqlens_q || !cu_seqlens_k || !out)
        return FSA_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return FSA_ERROR_INVALID_VALUE;
    const int32_t G = num_heads_q / num_heads_kv;
    if (num_splits == kSplitsBlockCentric) {
        if (dense || wl >= 0) return FSA_ERROR_INVALID_VALUE;       // windows have no such schedule
        if (!use_block_centric(G, num_splits, max_seqlen_q, total_q, num_heads_kv, topk))
            return FSA_ERROR_NOT_SUPPORTED;
    }
    if (!dense && wl < 0 && use_block_centric(G, num_splits, max_seqlen_q, total_q, num_heads_kv, topk))
        return prefill_bc(q, k, v, blk_idx, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                          max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, topk,
                          softmax_scale, wr >= 0, workspace, workspace_bytes, out, lse, stream);
    const PrefillPlan pl = plan_prefill(batch, max_seqlen_q, num_heads_q, num_heads_kv, num_splits);
    const size_t need = prefill_workspace(pl, total_q, num_heads_q, head_dim);
    if (pl.n_wg < 0) return FSA_ERROR_NOT_SUPPORTED;                // grid too large
    if (pl.splits > 1 && !groups_ok(((long long)total_q * num_heads_q + 3) / 4))
        return FSA_ERROR_NOT_SUPPORTED;                             // merge grid
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return FSA_ERROR_WORKSPACE;
    if (pl.n_wg == 0) return FSA_SUCCESS;
    PrefillPlan plo = pl;
    set_tile_order(plo, batch, num_heads_kv, max_seqlen_k, head_dim);

    fsa::SelFwdParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.blk_idx = blk_idx;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.total_q = total_q;
    p.total_k = total_k;
    p.batch = batch;
    p.Hq = num_heads_q;
    p.Hkv = num_heads_kv;
    p.G = num_heads_q / num_heads_kv;
    p.topk = dense ? 0 : topk;
    p.wl = wl;
    p.wr = wr;
    p.dense = dense ? 1 : 0;
    p.num_splits = pl.splits;
    p.T = pl.T;
    p.mtiles = pl.mtiles;
    p.tiles_per_seq = pl.tiles_per_seq;
    p.n_wg = plo.n_wg;
    p.head_major = plo.head_major;
    p.ring = fsa::sel_attn_fwd_ring(head_dim, pl.T, p.topk);
    p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    if (fsa::sel_attn_fwd_lds_bytes(head_dim, pl.T, p.topk, p.ring) > 160 * 1024)
        return FSA_ERROR_NOT_SUPPORTED;
    p.scale_log2 = resolve_scale(softmax_scale, head_dim) * fsa::kLog2e;
    const size_t rows = (size_t)total_q * num_heads_q;
    if (pl.splits > 1) {
        p.part_o = static_cast<float*>(workspace);
        p.part_lse = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                              align_up((size_t)pl.splits * rows * head_dim * 4));
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e = head_dim == 64 ? fsa::launch_sel_attn_fwd<64>(p, s)
                                  : fsa::launch_sel_attn_fwd<128>(p, s);
    if (e != hipSuccess) return FSA_ERROR_LAUNCH;
    if (pl.splits > 1) {
        fsa::MergeParams m{};
        m.part_o = p.part_o;
        m.part_lse = p.part_lse;
        m.out = p.out;
        m.lse = lse;
        m.nrows = (int64_t)rows;
        m.nparts = pl.splits;
        m.lse_mode = 0;
        m.Hq = num_heads_q;
        m.ntok = total_q;
        m.ntok_live = cu_seqlens_q + batch;
        e = fsa::launch_lse_merge(m, head_dim, s);
        if (e != hipSuccess) return FSA_ERROR_LAUNCH;
    }
    return FSA_SUCCESS;
}


extern "C" {

const char* fsa_status_string(fsa_status_t status) {
    // Callers may pass any integer; reading it as an int keeps out-of-range
    // codes defined (a load of an enum outside its values is not).
    static_assert(sizeof(fsa_status_t) == sizeof(int), "status is passed as an int");
    int code;
    std::memcpy(&code, &status, sizeof code);
    switch (code) {
        case FSA_SUCCESS: return "FSA_SUCCESS";
        case FSA_ERROR_INVALID_VALUE: return "FSA_ERROR_INVALID_VALUE";
        case FSA_ERROR_NOT_SUPPORTED: return "FSA_ERROR_NOT_SUPPORTED";
        case FSA_ERROR_WORKSPACE: return "FSA_ERROR_WORKSPACE";
        case FSA_ERROR_LAUNCH: return "FSA_ERROR_LAUNCH";
    }
    return "FSA_ERROR_UNKNOWN";
}

int32_t fsa_abi_version(void) { return FSA_ABI_VERSION; }

fsa_status_t fsa_wait_timeouts(uint32_t* count, int32_t reset) {
    if (count == nullptr) return FSA_ERROR_INVALID_VALUE;
    unsigned int a = 0, b = 0;
    (void)hipGetLastError();
    if (fsa::sel_attn_fwd_wait_timeouts(&a, reset != 0) != hipSuccess ||
        fsa::sel_attn_bwd_wait_timeouts(&b, reset != 0) != hipSuccess)
        return FSA_ERROR_LAUNCH;
    *count = a + b;
    return FSA_SUCCESS;
}

fsa_status_t fsa_set_wait_poll_limit(int32_t polls) {
    if (polls < 0) return FSA_ERROR_INVALID_VALUE;
    g_spin_limit.store(polls == 0 ? fsa::kDefaultSpinLimit : polls, std::memory_order_relaxed);
    return FSA_SUCCESS;
}

size_t fsa_selected_attn_fwd_workspace_size(int32_t batch, int64_t total_q, int32_t max_seqlen_q,
                                             int32_t max_seqlen_k, int32_t num_heads_q,
                                             int32_t num_heads_kv, int32_t head_dim,
                                             int32_t block_size, int32_t topk, int32_t num_splits) {
    if (total_q < 0 || max_seqlen_k < 0) return 0;
    if (check_prefill_shape(batch, max_seqlen_q, num_heads_q, num_heads_kv, head_dim, block_size,
                            topk, num_splits) != FSA_SUCCESS)
        return 0;
    max_seqlen_q = cap_len(max_seqlen_q, total_q);
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return 0;
    if (use_block_centric(num_heads_q / num_heads_kv, num_splits, max_seqlen_q, total_q,
                          num_heads_kv, topk))
        return bc_layout(batch, total_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, topk)
            .total;
    if (num_splits < 0) return 0;                 // a forced schedule the call would reject
    const PrefillPlan pl = plan_prefill(batch, max_seqlen_q, num_heads_q, num_heads_kv, num_splits);
    return prefill_workspace(pl, total_q, num_heads_q, head_dim);
}

fsa_status_t fsa_selected_attn_fwd(const void* q, const void* k, const void* v,
                                   const int32_t* blk_idx, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int32_t batch, int64_t total_q,
                                   int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int32_t block_size, int32_t topk, float softmax_scale,
                                   int32_t causal, int32_t num_splits, void* workspace,
                                   size_t workspace_bytes, void* out, float* lse, void* stream) {
    return prefill_impl(q, k, v, blk_idx, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                        max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                        block_size, topk, softmax_scale, -1, causal ? 0 : -1, false, num_splits,
                        workspace, workspace_bytes, out, lse, stream);
}

size_t fsa_sliding_window_fwd_workspace_size(int32_t batch, int64_t total_q,
                                             int32_t max_seqlen_q, int32_t num_heads_q,
                                             int32_t num_heads_kv, int32_t head_dim,
                                             int32_t num_splits) {
    if (total_q < 0 || num_splits < 0) return 0;
    if (check_prefill_shape(batch, max_seqlen_q, num_heads_q, num_heads_kv, head_dim,
                            fsa::kBlockKeys, 1, num_splits) != FSA_SUCCESS)
        return 0;
    max_seqlen_q = cap_len(max_seqlen_q, total_q);
    const PrefillPlan pl = plan_prefill(batch, max_seqlen_q, num_heads_q, num_heads_kv, num_splits);
    return prefill_workspace(pl, total_q, num_heads_q, head_dim);
}

fsa_status_t fsa_sliding_window_fwd(const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int64_t total_q, int64_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    int32_t window_left, int32_t window_right,
                                    float softmax_scale, int32_t num_splits, void* workspace,
                                    size_t workspace_bytes, void* out, float* lse, void* stream) {
    if (window_left < -1 || window_right < -1 || max_seqlen_k < 0 || num_splits < 0)
        return FSA_ERROR_INVALID_VALUE;     // (windows have no block-centric schedule)
    // A left bound of at least max_seqlen_k keys reaches below key 0 for every
    // row (i + S_k - S_q - left <= S_k - 1 - left < 0), so it is the same as
    // no limit.  The right bound is passed on unchanged: when S_q > S_k a
    // right bound larger than S_k still cuts rows near the start, and every
    // kernel use of it is 64-bit.
    const int32_t wl = window_left > max_seqlen_k ? max_seqlen_k : window_left;
    return prefill_impl(q, k, v, nullptr, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                        max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                        fsa::kBlockKeys, 1, softmax_scale, wl, window_right, true, num_splits, workspace,
                        workspace_bytes, out, lse, stream);
}

int32_t fsa_topk_decode_auto_splits(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t topk) {
    if (check_decode_shape(batch, num_heads_q, num_heads_kv, 64, topk, 0) != FSA_SUCCESS) return 0;
    return decode_auto_splits(batch, num_heads_q, num_heads_kv, topk);
}

size_t fsa_topk_decode_workspace_size(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                      int32_t head_dim, int32_t topk, int32_t num_splits) {
    if (check_decode_shape(batch, num_heads_q, num_heads_kv, head_dim, topk, num_splits) !=
        FSA_SUCCESS)
        return 0;
    return decode_layout(batch, num_heads_q, num_heads_kv, head_dim, topk, num_splits).total;
}

fsa_status_t fsa_topk_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* tok_idx, const int32_t* block_table,
                             const int32_t* cache_seqlens, int32_t batch, int32_t num_heads_q,
                             int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
                             int32_t max_pages_per_seq, int32_t num_pages, int32_t topk,
                             float softmax_scale, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, void* stream) {
    return decode_impl(q, k_cache, v_cache, false, nullptr, nullptr, tok_idx, block_table,
                       cache_seqlens, batch, num_heads_q, num_heads_kv, head_dim, page_size,
                       max_pages_per_seq, num_pages, topk, softmax_scale, num_splits, workspace,
                       workspace_bytes, out, lse, stream);
}

fsa_status_t fsa_topk_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* tok_idx, const int32_t* block_table,
                                     const int32_t* cache_seqlens, int32_t batch,
                                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                     int32_t page_size, int32_t max_pages_per_seq,
                                     int32_t num_pages, int32_t topk, float softmax_scale,
                                     int32_t num_splits, void* out, float* lse, void* stream) {
    fsa_status_t st = check_decode_shape(batch, num_heads_q, num_heads_kv, head_dim, topk,
                                         num_splits);
    if (st != FSA_SUCCESS) return st;
    if (batch == 0) return FSA_SUCCESS;
    const DecodeLayout lay = decode_layout(batch, num_heads_q, num_heads_kv, head_dim, topk,
                                           num_splits);
    if (lay.total > kNoAllocScratchBytes) return FSA_ERROR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (lay.total > 0) {
        st = noalloc_scratch(&ws);
        if (st != FSA_SUCCESS) return st;
        ws_bytes = kNoAllocScratchBytes;
    }
    return decode_impl(q, k_cache, v_cache, false, nullptr, nullptr, tok_idx, block_table,
                       cache_seqlens, batch, num_heads_q, num_heads_kv, head_dim, page_size,
                       max_pages_per_seq, num_pages, topk, softmax_scale, num_splits, ws,
                       ws_bytes, out, lse, stream);
}

fsa_status_t fsa_topk_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                 const float* k_descale, const float* v_descale,
                                 const int32_t* tok_idx, const int32_t* block_table,
                                 const int32_t* cache_seqlens, int32_t batch, int32_t num_heads_q,
                                 int32_t num_heads_kv, int32_t head_dim, int32_t page_size,
                                 int32_t max_pages_per_seq, int32_t num_pages, int32_t topk,
                                 float softmax_scale, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse, void* stream) {
    return decode_impl(q, k_cache, v_cache, true, k_descale, v_descale, tok_idx, block_table,
                       cache_seqlens, batch, num_heads_q, num_heads_kv, head_dim, page_size,
                       max_pages_per_seq, num_pages, topk, softmax_scale, num_splits, workspace,
                       workspace_bytes, out, lse, stream);
}

struct BwdLayout {
    size_t dvec, counts, cursor, toks, kv_acc, total;
    int nb_max;
};

static BwdLayout bwd_layout(int32_t batch, int64_t total_q, int64_t total_k, int32_t max_seqlen_k,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t topk) {
    BwdLayout l{};
    l.nb_max = (int)(((long long)max_seqlen_k + fsa::kBlockKeys - 1) / fsa::kBlockKeys);
    if (l.nb_max < 1) l.nb_max = 1;
    size_t off = 0;
    l.dvec = off;
    off = align_up(off + (size_t)Hq * total_q * 4);
    l.counts = off;
    off = align_up(off + (size_t)batch * Hkv * (l.nb_max + 1) * 4);
    l.cursor = off;
    off = align_up(off + (size_t)batch * Hkv * l.nb_max * 4);
    l.toks = off;
    off = align_up(off + (size_t)total_q * Hkv * topk * 4);
    l.kv_acc = off;
    off = align_up(off + (size_t)total_k * Hkv * 2 * D * 4);
    l.total = off;
    return l;
}

static fsa_status_t check_bwd_shape(int32_t batch, int64_t total_q, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t bs, int32_t topk) {
    fsa_status_t st = check_prefill_shape(batch, max_seqlen_q, Hq, Hkv, D, bs, topk, 1);
    if (st != FSA_SUCCESS) return st;
    if (total_q < 0 || max_seqlen_k < 0) return FSA_ERROR_INVALID_VALUE;
    if (Hq / Hkv > kMaxGroupBackward) return FSA_ERROR_NOT_SUPPORTED;
    return FSA_SUCCESS;
}

size_t fsa_selected_attn_bwd_workspace_size(int32_t batch, int64_t total_q, int64_t total_k,
                                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                                            int32_t num_heads_q, int32_t num_heads_kv,
                                            int32_t head_dim, int32_t block_size, int32_t topk) {
    if (total_k < 0 ||
        check_bwd_shape(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                        head_dim, block_size, topk) != FSA_SUCCESS)
        return 0;
    max_seqlen_k = cap_len(max_seqlen_k, total_k);
    return bwd_layout(batch, total_q, total_k, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                      topk).total;
}

fsa_status_t fsa_selected_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                                   const float* lse, const void* dout, const int32_t* blk_idx,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t batch, int64_t total_q, int64_t total_k,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int32_t block_size, int32_t topk, float softmax_scale,
                                   int32_t causal, void* workspace, size_t workspace_bytes,
                                   void* dq, void* dk, void* dv, void* stream) {
    fsa_status_t st = check_bwd_shape(batch, total_q, max_seqlen_q, max_seqlen_k, num_heads_q,
                                      num_heads_kv, head_dim, block_size, topk);
    if (st != FSA_SUCCESS) return st;
    if (total_k < 0) return FSA_ERROR_INVALID_VALUE;
    if (total_q > INT32_MAX || total_k > INT32_MAX) return FSA_ERROR_NOT_SUPPORTED;
    max_seqlen_q = cap_len(max_seqlen_q, total_q);
    max_seqlen_k = cap_len(max_seqlen_k, total_k);
    if (batch == 0 || (total_q == 0 && total_k == 0)) return FSA_SUCCESS;
    if (!q || !k || !v || !out || !lse || !dout || !blk_idx || !cu_seqlens_q || !cu_seqlens_k ||
        !dq || !dk || !dv)
        return FSA_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return FSA_ERROR_INVALID_VALUE;
    const BwdLayout lay = bwd_layout(batch, total_q, total_k, max_seqlen_k, num_heads_q,
                                     num_heads_kv, head_dim, topk);
    if (workspace == nullptr || workspace_bytes < lay.total ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return FSA_ERROR_WORKSPACE;
    const int G = num_heads_q / num_heads_kv;
    int T = fsa::sel_attn_bwd_rows_per_tile() / G;
    if (T > 64) T = 64;
    if (T < 1) T = 1;
    const int dq_ring = fsa::sel_attn_bwd_dq_ring(head_dim, T, topk);
    if (dq_ring < 2) return FSA_ERROR_NOT_SUPPORTED;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    fsa::SelBwdParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<const uint16_t*>(out);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.blk_idx = blk_idx;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    p.dvec = reinterpret_cast<float*>(ws + lay.dvec);
    p.counts = reinterpret_cast<int32_t*>(ws + lay.counts);
    p.cursor = reinterpret_cast<int32_t*>(ws + lay.cursor);
    p.toks = reinterpret_cast<int32_t*>(ws + lay.toks);
    p.kv_acc = reinterpret_cast<float*>(ws + lay.kv_acc);
    p.total_q = total_q;
    p.total_k = total_k;
    p.batch = batch;
    p.Hq = num_heads_q;
    p.Hkv = num_heads_kv;
    p.G = G;
    p.topk = topk;
    p.causal = causal ? 1 : 0;
    p.nb_max = lay.nb_max;
    {
        // a block is split only when it has more steps of 32 rows than one
        // part takes (>= 64 steps, at most 32 parts); the parts meet in fp32
        // atomics
        const long long tpc = 32 / G;          // whole tokens per step of 32 rows
        const long long max_steps = ((long long)max_seqlen_q + tpc - 1) / tpc;
        long long np = (max_steps + 63) / 64;
        if (np > 32) np = 32;
        if (np < 1) np = 1;
        p.nparts = (int)np;
        p.part_steps = (int)((max_steps + np - 1) / np);
        if (p.part_steps < 1) p.part_steps = 1;
    }
    p.T = T;
    p.ring = dq_ring;
    p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    const int chunk = fsa::sel_attn_bwd_index_chunk();
    p.nchunk_q = (int)(((long long)max_seqlen_q + chunk - 1) / chunk);
    if (p.nchunk_q < 1) p.nchunk_q = 1;
    p.mtiles = (T * G + 15) / 16;
    p.tiles_per_seq = (int)(((long long)max_seqlen_q + T - 1) / T);
    if (p.tiles_per_seq < 1) p.tiles_per_seq = 1;
    {
        const long long units = (long long)batch * num_heads_kv;
        if (!groups_ok(((long long)total_q * num_heads_q + 15) / 16) ||
            !groups_ok(units * p.nchunk_q) || !groups_ok(units * lay.nb_max * p.nparts) ||
            !groups_ok(units * p.tiles_per_seq))
            return FSA_ERROR_NOT_SUPPORTED;
    }
    p.scale = resolve_scale(softmax_scale, head_dim);
    p.scale_log2 = p.scale * fsa::kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (fsa::launch_sel_attn_bwd(p, head_dim, s) != hipSuccess) return FSA_ERROR_LAUNCH;
    return FSA_SUCCESS;
}

size_t fsa_block_select_workspace_size(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_kv,
                                       int32_t head_dim, int32_t kernel_size, int32_t kernel_stride) {
    if (check_select(batch, 0, max_seqlen_k, num_heads_kv, num_heads_kv, head_dim, kernel_size,
                     kernel_stride, fsa::kBlockKeys, 1, 0, 0) != FSA_SUCCESS)
        return 0;
    const SelectPlan pl = plan_select(0, max_seqlen_k, num_heads_kv, num_heads_kv);
    return align_up((size_t)batch * pl.ncmp_max * num_heads_kv * head_dim * 2);
}

fsa_status_t fsa_block_select(const void* q, const void* k, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int64_t total_q,
                              int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                              int32_t kernel_size, int32_t kernel_stride, int32_t block_size,
                              int32_t topk, int32_t init_blocks, int32_t local_blocks,
                              float softmax_scale, void* workspace, size_t workspace_bytes,
                              int32_t* blk_idx, void* stream) {
    fsa_status_t st = check_select(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                                   head_dim, kernel_size, kernel_stride, block_size, topk,
                                   init_blocks, local_blocks);
    if (st != FSA_SUCCESS) return st;
    if (total_q < 0 || total_k < 0) return FSA_ERROR_INVALID_VALUE;
    if (total_q > INT32_MAX || total_k > INT32_MAX) return FSA_ERROR_NOT_SUPPORTED;
    max_seqlen_q = cap_len(max_seqlen_q, total_q);
    max_seqlen_k = cap_len(max_seqlen_k, total_k);
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FSA_SUCCESS;   // nothing to do
    if (!q || !k || !cu_seqlens_q || !cu_seqlens_k || !blk_idx) return FSA_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k)) return FSA_ERROR_INVALID_VALUE;
    const SelectPlan pl = plan_select(max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv);
    if (pl.T < 1) return FSA_ERROR_NOT_SUPPORTED;
    if (!groups_ok((long long)batch * num_heads_kv * pl.tiles_per_seq) ||
        !groups_ok(((long long)batch * pl.ncmp_max * num_heads_kv * (head_dim / 8) + 255) / 256))
        return FSA_ERROR_NOT_SUPPORTED;
    const size_t need = fsa_block_select_workspace_size(batch, max_seqlen_k, num_heads_kv, head_dim,
                                                        kernel_size, kernel_stride);
    if (pl.ncmp_max > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return FSA_ERROR_WORKSPACE;

    fsa::BlockSelectParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.cmp = static_cast<uint16_t*>(workspace);
    p.blk_idx = blk_idx;
    p.total_q = total_q;
    p.total_k = total_k;
    p.batch = batch;
    p.Hq = num_heads_q;
    p.Hkv = num_heads_kv;
    p.G = num_heads_q / num_heads_kv;
    p.topk = topk;
    p.init = init_blocks;
    p.local = local_blocks;
    p.ncmp_max = pl.ncmp_max;
    p.nb_max = pl.nb_max;
    p.T = pl.T;
    p.mtiles = pl.mtiles;
    p.tiles_per_seq = pl.tiles_per_seq;
    p.scale_log2 = resolve_scale(softmax_scale, head_dim) * fsa::kLog2e;
    (void)hipGetLastError();
    if (fsa::launch_block_select(p, head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
        return FSA_ERROR_LAUNCH;
    return FSA_SUCCESS;
}

}  // extern "C"
