// sel_attn_fwd.hip -- top-k selected block-sparse attention forward (prefill), gfx950.
//
// What it computes (FSA page: NSA selected attention with block_size / topk;
// flash-attention-npu page, flash_attn_varlen_func docstring: varlen layout,
// GQA mapping, bottom-right causal mask, zero rows, natural-log LSE): every
// query row of (token t, q head h) attends to the keys of the blocks listed
// in blk_idx[t, h / G, :], read as a set, under the bottom-right causal mask.
//
// Schedule.  One workgroup owns a tile of T consecutive query tokens of one
// sequence and one kv head g.  All T*G query rows of the tile are packed
// GQA-first into 16-row MFMA tiles ("m-tiles": row r = token r / G, head
// r % G), so the query group forms the MFMA M dimension.  The workgroup
// builds, in LDS, the ascending union of the blocks its tokens selected
// together with a per-block bitmask of the selecting tokens, then streams the
// union: each K/V block is loaded once (coalesced 16-byte loads), staged in
// LDS double-buffered (K row-major, V transposed), and consumed by every
// m-tile that contains a selecting token.  Rows whose token did not select
// the block are masked to -inf, exactly like causally masked keys.
//
// Per m-tile and block the contraction runs transposed, S^T = K * Q^T with
// v_mfma_f32_16x16x32_bf16: the key index is the MFMA row, the query row the
// column.  The accumulator layout of S^T leaves each lane holding, for one
// query row, exactly the keys that lane must supply to the P^T operand of
// O^T = V^T * P^T, so P never leaves registers.  Online softmax runs in the
// log2 domain (scale folded with log2 e); a row's running max is shared by
// its four lanes through two cross-lane exchanges per block.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

constexpr int kSelWaves = 8;                       // waves per workgroup
constexpr int kSelThreads = kSelWaves * 64;
constexpr int kSelMtPerWave = 2;                   // m-tiles owned by each wave
constexpr int kSelWin = 512;                       // blocks per union-building window


// LDS layout (bytes) for head dim D.
template <int D>
struct SelLds {
    static constexpr int kK = kBlockKeys * D * 2;        // K tile, row-major, swizzled
    static constexpr int kVt = D * kBlockKeys * 2;       // V^T tile, swizzled
    static constexpr int kStage = kK + kVt;
    static constexpr int kMasks = 2 * kStage;            // u64 [kSelWin]
    static constexpr int kUMask = kMasks + kSelWin * 8;  // u64 [kSelWin]
    static constexpr int kUList = kUMask + kSelWin * 8;  // i32 [kSelWin]
    static constexpr int kCount = kUList + kSelWin * 4;  // i32
    static constexpr int kEnt = kCount + 16;             // i32 [T*topk]
    static size_t bytes(int T, int topk) { return (size_t)kEnt + (size_t)T * topk * 4; }
};

template <int D>
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
    constexpr int NCH = D / 8;
    return key * (D * 2) + ((chunk ^ (key & (NCH - 1))) << 4);
}
__device__ __forceinline__ int vt_lds_off(int d, int chunk) {
    return d * (kBlockKeys * 2) + ((chunk ^ (d & 7)) << 4);
}

template <int D>
__global__ void __launch_bounds__(kSelThreads)
sel_attn_fwd_kernel(const SelFwdParams p) {
    constexpr int NCH = D / 8;                  // 16-byte chunks per K/V row
    constexpr int KS = D / 32;                  // MFMA k-steps over the head dim
    constexpr int DT = D / 16;                  // 16-wide tiles of the head dim
    constexpr int KCH = (kBlockKeys * NCH) / kSelThreads;   // K chunks per thread
    constexpr int VSB = 16 * NCH;               // 4-key x 8-dim V sub-blocks per block
    static_assert(KCH >= 1 && (kBlockKeys * NCH) % kSelThreads == 0, "K staging split");
    static_assert(VSB <= kSelThreads, "V staging split");
    using L = SelLds<D>;

    extern __shared__ __align__(16) uint8_t smem[];
    unsigned long long* s_masks = reinterpret_cast<unsigned long long*>(smem + L::kMasks);
    unsigned long long* s_umask = reinterpret_cast<unsigned long long*>(smem + L::kUMask);
    int* s_ulist = reinterpret_cast<int*>(smem + L::kUList);
    int* s_count = reinterpret_cast<int*>(smem + L::kCount);
    int* s_ent = reinterpret_cast<int*>(smem + L::kEnt);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;        // MFMA column = query row within the m-tile
    const int lg = lane >> 4;        // lane group 0..3

    // ---- which tile: heavy (late) tiles first, tiles of one (seq, kv head) on one XCD
    int w = xcd_remap(blockIdx.x, p.n_wg);
    const int j = p.tiles_per_seq - 1 - (w % p.tiles_per_seq);
    w /= p.tiles_per_seq;
    const int split = w % p.num_splits;
    w /= p.num_splits;
    const int g = w % p.Hkv;
    const int b = w / p.Hkv;

    int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    int64_t k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    q1 = q1 < p.total_q ? q1 : p.total_q;
    q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
    k1 = k1 < p.total_k ? k1 : p.total_k;
    k0 = k0 < 0 ? 0 : (k0 < k1 ? k0 : k1);
    const int Sq = (int)(q1 - q0);
    const int Sk = (int)(k1 - k0);
    const int tok0 = j * p.T;
    if (tok0 >= Sq) return;                     // whole workgroup: past the sequence end
    const int ntok = (Sq - tok0) < p.T ? (Sq - tok0) : p.T;
    const int off = Sk - Sq;                    // bottom-right alignment shift
    const int nblk = (Sk + kBlockKeys - 1) / kBlockKeys;
    int nb_range = nblk;                        // blocks that can hold a visible key
    if (p.causal) {
        const int last_key = tok0 + ntok - 1 + off;
        nb_range = last_key < 0 ? 0 : (last_key / kBlockKeys + 1);
        nb_range = nb_range < nblk ? nb_range : nblk;
    }
    const int topk = p.topk;
    const int G = p.G;

    // ---- the tile's lists -> LDS, dropping ids outside the range and fully-future blocks
    const int nent = ntok * topk;
    for (int e = tid; e < nent; e += kSelThreads) {
        const int tl = e / topk;
        const int slot = e - tl * topk;
        int id = p.blk_idx[((q0 + tok0 + tl) * p.Hkv + g) * (int64_t)topk + slot];
        bool ok = id >= 0 && id < nb_range;
        if (ok && p.causal) ok = id * kBlockKeys <= tok0 + tl + off;
        s_ent[e] = ok ? id : -1;
    }

    // ---- per-lane row bookkeeping for the owned m-tiles
    float m_run[kSelMtPerWave], l_run[kSelMtPerWave];
    f32x4_t acc[kSelMtPerWave][DT];
    u32x4_t qf[kSelMtPerWave][KS];
    unsigned long long mt_tok[kSelMtPerWave];   // tokens covered by the m-tile
    int row_tl[kSelMtPerWave], row_lim[kSelMtPerWave];
#pragma unroll
    for (int t = 0; t < kSelMtPerWave; ++t) {
        const int mt = wave * kSelMtPerWave + t;
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int row = mt * 16 + lr;
        const int tl = row / G;
        const int hh = row - tl * G;
        const bool valid = mt < p.mtiles && tl < ntok;
        row_tl[t] = valid ? tl : 63;
        // keys with local index < row_lim are visible to this row
        int lim = Sk;
        if (p.causal) {
            const int c = tok0 + tl + off + 1;
            lim = c < lim ? c : lim;
        }
        row_lim[t] = valid ? lim : 0;
        const uint16_t* qrow = p.q + ((q0 + tok0 + tl) * p.Hq + g * G + hh) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[t][s] = valid ? *reinterpret_cast<const u32x4_t*>(qrow + s * 32 + lg * 8)
                             : u32x4_t{0u, 0u, 0u, 0u};
        }
        unsigned long long mk = 0ull;
        if (mt < p.mtiles) {
            const int t_first = (mt * 16) / G;
            int t_last = (mt * 16 + 15) / G;
            t_last = t_last < ntok - 1 ? t_last : ntok - 1;
            for (int x = t_first; x <= t_last; ++x) mk |= 1ull << x;
        }
        mt_tok[t] = mk;
    }

    // ---- staging of one K/V block: global -> registers -> LDS (K row-major, V transposed)
    u32x4_t kreg[KCH];
    u32x4_t vreg[4];
    const uint16_t* kbase = p.k + (k0 * p.Hkv + g) * (int64_t)D;
    const uint16_t* vbase = p.v + (k0 * p.Hkv + g) * (int64_t)D;
    const int64_t krow_stride = (int64_t)p.Hkv * D;

    auto issue_loads = [&](int blk) {
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int idx = tid + kSelThreads * r;
            const int key = idx / NCH, c = idx % NCH;
            const int krow = blk * kBlockKeys + key;
            kreg[r] = krow < Sk ? *reinterpret_cast<const u32x4_t*>(kbase + krow * krow_stride + c * 8)
                                : u32x4_t{0u, 0u, 0u, 0u};
        }
        if (tid < VSB) {
            const int c = tid % NCH, kg = tid / NCH;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int krow = blk * kBlockKeys + 4 * kg + r;
                vreg[r] = krow < Sk ? *reinterpret_cast<const u32x4_t*>(vbase + krow * krow_stride + c * 8)
                                    : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto write_stage = [&](int buf) {
        uint8_t* kb = smem + buf * L::kStage;
        uint8_t* vt = kb + L::kK;
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int idx = tid + kSelThreads * r;
            const int key = idx / NCH, c = idx % NCH;
            *reinterpret_cast<u32x4_t*>(kb + k_lds_off<D>(key, c)) = kreg[r];
        }
        if (tid < VSB) {
            const int c = tid % NCH, kg = tid / NCH;
            // keys 4kg..4kg+3 = 32*ks + 16*h + 4*gg + i  ->  position 32*ks + 8*gg + 4*h + i
            const int ks = kg >> 3, h = (kg >> 2) & 1, gg = kg & 3;
            const int pchunk = 4 * ks + gg;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t w0 = vreg[0][x], w1 = vreg[1][x], w2 = vreg[2][x], w3 = vreg[3][x];
                const u32x2_t lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
                const u32x2_t hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
                const int d0 = c * 8 + 2 * x;
                *reinterpret_cast<u32x2_t*>(vt + vt_lds_off(d0, pchunk) + 8 * h) = lo;
                *reinterpret_cast<u32x2_t*>(vt + vt_lds_off(d0 + 1, pchunk) + 8 * h) = hi;
            }
        }
    };

    // ---- one m-tile against one staged block
    auto compute = [&](int t, int buf, int blk, unsigned long long bmask) {
        const uint8_t* kb = smem + buf * L::kStage;
        const uint8_t* vt = kb + L::kK;
        f32x4_t st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kb + k_lds_off<D>(kt * 16 + lr, 4 * s + lg));
                st[kt] = mfma_16x16x32(a, qf[t][s], st[kt]);
            }
        }
        // mask: token did not select the block, causal limit, sequence end
        const int lim = ((bmask >> row_tl[t]) & 1ull) ? row_lim[t] - blk * kBlockKeys : 0;
        float x[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kt * 16 + lg * 4 + i;
                const float v = key < lim ? st[kt][i] * p.scale_log2 : -INFINITY;
                x[kt * 4 + i] = v;
                mloc = fmaxf(mloc, v);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run[t], mloc);
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[t] - msub);
        m_run[t] = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x[e] = fast_exp2(x[e] - msub);
            lsum += x[e];
        }
        l_run[t] = l_run[t] * alpha + lsum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[t][dt] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4_t pb = {pack_bf16x2(x[8 * ks + 0], x[8 * ks + 1]),
                                pack_bf16x2(x[8 * ks + 2], x[8 * ks + 3]),
                                pack_bf16x2(x[8 * ks + 4], x[8 * ks + 5]),
                                pack_bf16x2(x[8 * ks + 6], x[8 * ks + 7])};
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vt + vt_lds_off(dt * 16 + lr, 4 * ks + lg));
                acc[t][dt] = mfma_16x16x32(a, pb, acc[t][dt]);
            }
        }
    };

    __syncthreads();   // s_ent ready

    for (int win_lo = 0; win_lo < nb_range; win_lo += kSelWin) {
        const int win_n = (nb_range - win_lo) < kSelWin ? (nb_range - win_lo) : kSelWin;
        for (int x = tid; x < kSelWin; x += kSelThreads) s_masks[x] = 0ull;
        __syncthreads();
        for (int e = tid; e < nent; e += kSelThreads) {
            const int id = s_ent[e];
            if (id >= win_lo && id < win_lo + win_n) atomicOr(&s_masks[id - win_lo], 1ull << (e / topk));
        }
        __syncthreads();
        if (wave == 0) {      // ascending compaction of the non-empty blocks
            int n = 0;
            for (int c = 0; c < win_n; c += 64) {
                const int x = c + lane;
                const unsigned long long m = x < win_n ? s_masks[x] : 0ull;
                const unsigned long long bal = __ballot(m != 0ull);
                if (m != 0ull) {
                    const int pos = n + __popcll(bal & ((1ull << lane) - 1ull));
                    s_ulist[pos] = win_lo + x;
                    s_umask[pos] = m;
                }
                n += __popcll(bal);
            }
            if (lane == 0) s_count[0] = n;
        }
        __syncthreads();
        const int n_u = s_count[0];
        const int u_beg = (int)(((long long)n_u * split) / p.num_splits);
        const int u_end = (int)(((long long)n_u * (split + 1)) / p.num_splits);
        if (u_beg < u_end) {
            issue_loads(s_ulist[u_beg]);
            write_stage(0);
            __syncthreads();
            for (int u = u_beg; u < u_end; ++u) {
                const int buf = (u - u_beg) & 1;
                const bool has_next = u + 1 < u_end;
                if (has_next) issue_loads(s_ulist[u + 1]);
                const int blk = s_ulist[u];
                const unsigned long long bm = s_umask[u];
#pragma unroll
                for (int t = 0; t < kSelMtPerWave; ++t) {
                    if (bm & mt_tok[t]) compute(t, buf, blk, bm);
                }
                if (has_next) write_stage(buf ^ 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: normalise, write O (bf16) and LSE, or the split partials
#pragma unroll
    for (int t = 0; t < kSelMtPerWave; ++t) {
        const int mt = wave * kSelMtPerWave + t;
        if (mt >= p.mtiles) continue;
        float l = l_run[t];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int row = mt * 16 + lr;
        const int tl = row / G;
        const int hh = row - tl * G;
        if (tl >= ntok) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse_v = l > 0.f ? (m_run[t] + __log2f(l)) * kLn2 : -INFINITY;
        const int64_t tok = q0 + tok0 + tl;
        const int head = g * G + hh;
        const int64_t orow = tok * p.Hq + head;
        if (p.num_splits == 1) {
            uint16_t* o = p.out + orow * D + lg * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x2_t pk = {pack_bf16x2(acc[t][dt][0] * inv, acc[t][dt][1] * inv),
                                    pack_bf16x2(acc[t][dt][2] * inv, acc[t][dt][3] * inv)};
                *reinterpret_cast<u32x2_t*>(o + dt * 16) = pk;
            }
            if (p.lse != nullptr && lg == 0) p.lse[(int64_t)head * p.total_q + tok] = lse_v;
        } else {
            const int64_t prow = (int64_t)split * p.total_q * p.Hq + orow;
            float* o = p.part_o + prow * D + lg * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                *reinterpret_cast<f32x4_t*>(o + dt * 16) = acc[t][dt] * inv;
            }
            if (lg == 0) p.part_lse[prow] = lse_v;
        }
    }
}

// Launch helpers (host side).
template <int D>
hipError_t launch_sel_attn_fwd(const SelFwdParams& p, hipStream_t stream) {
    const size_t lds = SelLds<D>::bytes(p.T, p.topk);
    static bool attr_set = false;   // idempotent; racing threads set the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sel_attn_fwd_kernel<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(sel_attn_fwd_kernel<D>, dim3(p.n_wg), dim3(kSelThreads), lds, stream, p);
    return hipGetLastError();
}

template hipError_t launch_sel_attn_fwd<64>(const SelFwdParams&, hipStream_t);
template hipError_t launch_sel_attn_fwd<128>(const SelFwdParams&, hipStream_t);

size_t sel_attn_fwd_lds_bytes(int D, int T, int topk) {
    return D == 64 ? SelLds<64>::bytes(T, topk) : SelLds<128>::bytes(T, topk);
}

}  // namespace fsa
