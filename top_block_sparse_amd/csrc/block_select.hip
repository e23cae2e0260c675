// block_select.hip -- block-index producer for selected attention, gfx950.
//
// What it computes (FSA page, quick start: the compressed view of the keys --
// kernel_size 32, kernel_stride 16 -- from which the selection of block_size
// 64 blocks, topk, init_blocks and local_blocks is made; the pages give these
// parameters only, so each step is the plain reading stated here):
//   1. compressed keys: window j of a sequence covers keys [16j, 16j + 32)
//      (windows exist while they fit in the sequence); its summary is the
//      mean of its 32 keys per kv head, rounded to bf16;
//   2. compressed attention: row (token i, q head h) sees window j when the
//      whole window is in its causal past, 16j + 31 <= i + S_k - S_q;
//      p_j = softmax over those windows of scale * <q, c_j>;
//   3. block importance: a window's probability is spread evenly over its
//      keys, block b collects the mass of its 64 keys, summed over the q
//      heads of the kv head's group: windows 4b, 4b+1, 4b+2 lie inside
//      block b, window 4b+3 straddles b and b+1 (half each);
//   4. selection: blocks 0 .. init-1, then the local blocks qb, qb-1, ...,
//      then the candidates [init, qb - local + 1) of largest importance (ties
//      to the smaller block), -1 pads; qb = floor((i + S_k - S_q) / 64).
//
// Kernels:
//   cmp_keys_kernel   one thread per (sequence, window, kv head, 8 dims):
//                     fp32 sum of 32 bf16 keys, times 1/32, RNE to bf16;
//   block_select_kernel  a workgroup per (T tokens, kv head): each of 8 waves
//                     owns one 16-row m-tile of the T*G query rows
//                     (GQA-packed like the prefill) and runs S^T = C Q^T with
//                     v_mfma_f32_16x16x32_bf16 over the visible windows in
//                     two passes -- row max and sum, then probabilities --
//                     from chunks of 64 window summaries staged once in LDS,
//                     adding block masses into an LDS table [T][blocks];
//                     then the forced blocks are listed and the rest picked
//                     by repeated argmax: with at most 128 candidates per
//                     token, four tokens per wave (one per 16-lane row, the
//                     candidates in registers, a DPP row maximum per pick),
//                     otherwise one wave per token over the LDS table.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

namespace {

constexpr int kSelBlock = 64;          // keys per selection block
constexpr int kCmpSize = 32;           // keys per compressed window
constexpr int kCmpStride = 16;         // window stride
constexpr int kSelectWaves = 8;
constexpr int kSelectThreads = kSelectWaves * 64;
constexpr int kWinChunk = 64;          // windows per MFMA chunk (4 key tiles of 16)
constexpr int kPickRegs = 8;           // register-held candidates per lane in the row-wise selection

struct Bounds {
    int64_t q0, k0;
    int Sq, Sk;
};

__device__ __forceinline__ Bounds seq_bounds(const int32_t* cu_q, const int32_t* cu_k, int b,
                                             int64_t total_q, int64_t total_k) {
    int64_t q0 = cu_q[b], q1 = cu_q[b + 1];
    int64_t k0 = cu_k[b], k1 = cu_k[b + 1];
    q1 = q1 < total_q ? q1 : total_q;
    q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
    k1 = k1 < total_k ? k1 : total_k;
    k0 = k0 < 0 ? 0 : (k0 < k1 ? k0 : k1);
    return Bounds{q0, k0, (int)(q1 - q0), (int)(k1 - k0)};
}

__device__ __forceinline__ int n_windows(int Sk) {
    return Sk >= kCmpSize ? (Sk - kCmpSize) / kCmpStride + 1 : 0;
}

__device__ __forceinline__ uint32_t rne_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// sum over aligned groups of n lanes (n = 1, 2, 4, 8 or 16) of a 16-lane row;
// every lane of a group ends with the group's sum
__device__ __forceinline__ float group_sum(float x, int n) {
    if (n >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    if (n >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    if (n >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    if (n >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

#define FSA_DPP_U64(v, ctrl)                                                                       \
    ((((unsigned long long)(uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((v) >> 32), ctrl, \
                                                                 0xF, 0xF, false)) << 32) |       \
     (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v), ctrl, 0xF, 0xF, false))

// maximum of a 64-bit key over each 16-lane row (every lane of the row gets
// it): quad swaps, then the half-row and row mirrors
__device__ __forceinline__ unsigned long long row_max_u64(unsigned long long x) {
    auto pick = [](unsigned long long a, unsigned long long b) { return a > b ? a : b; };
    x = pick(x, FSA_DPP_U64(x, 0xB1));
    x = pick(x, FSA_DPP_U64(x, 0x4E));
    x = pick(x, FSA_DPP_U64(x, 0x141));
    x = pick(x, FSA_DPP_U64(x, 0x140));
    return x;
}
#undef FSA_DPP_U64

// wave-wide maximum of a 64-bit key: the row maximum, then the gfx950
// permlane swaps across rows (all VALU; no LDS round trips)
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
    auto pick = [](unsigned long long a, unsigned long long b) { return a > b ? a : b; };
    x = row_max_u64(x);
    {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
        x = pick(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
        x = pick(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    return uniform_u64(x);
}

}  // namespace

// ---- 1. compressed keys [batch][ncmp_max][Hkv][D] bf16 (zeros past a sequence's windows)
template <int D>
__global__ void __launch_bounds__(256) cmp_keys_kernel(const BlockSelectParams p) {
    constexpr int CPR = D / 8;                         // 8-dim chunks per row
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)p.batch * p.ncmp_max * p.Hkv * CPR;
    if (x >= n) return;
    const int cc = (int)(x % CPR);
    int64_t r = x / CPR;
    const int g = (int)(r % p.Hkv);
    r /= p.Hkv;
    const int j = (int)(r % p.ncmp_max);
    const int b = (int)(r / p.ncmp_max);
    const Bounds sb = seq_bounds(p.cu_q, p.cu_k, b, p.total_q, p.total_k);
    u32x4_t outv = {0u, 0u, 0u, 0u};
    if (j < n_windows(sb.Sk)) {                          // (j < ncmp_max by the grid)
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        const uint16_t* kr = p.k + ((sb.k0 + (int64_t)j * kCmpStride) * p.Hkv + g) * (int64_t)D + cc * 8;
        for (int t = 0; t < kCmpSize; ++t) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + (int64_t)t * p.Hkv * D);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_lo(v[e]);
                acc[2 * e + 1] += bf16_hi(v[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            outv[e] = rne_bf16_bits(acc[2 * e] * (1.f / kCmpSize)) |
                      (rne_bf16_bits(acc[2 * e + 1] * (1.f / kCmpSize)) << 16);
    }
    *reinterpret_cast<u32x4_t*>(p.cmp + (((int64_t)b * p.ncmp_max + j) * p.Hkv + g) * D + cc * 8) = outv;
}

// ---- 2. compressed attention, block importance and selection
// LDS: the importance table [T][nb_max] fp32, then two buffers of one chunk
// of 64 window summaries in MFMA A-operand order -- fragment (kt, s), 1 KiB,
// lane l's 16 bytes = C[16kt + l%16][32s + 8(l/16) .. +8] -- so every operand
// read is one contiguous wave read.  The chunk is loaded once per workgroup
// (all waves share it), the next one while the current one is used.
// Six waves per SIMD (80 VGPRs): three workgroups share a CU, as the LDS
// allows; at the compiler's own choice of 92 VGPRs only two fit.
template <int D>
__global__ void __launch_bounds__(kSelectThreads, 6) block_select_kernel(const BlockSelectParams p) {
    constexpr int KS = D / 32;
    constexpr int CPR = D / 8;                                   // 16-byte pieces per window
    constexpr int kChunkBytes = kWinChunk * D * 2;
    constexpr int NL = kWinChunk * CPR / kSelectThreads;         // pieces per thread per chunk
    static_assert(NL * kSelectThreads == kWinChunk * CPR, "chunk staging");
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    int w = xcd_remap(blockIdx.x, (int)gridDim.x);
    const int jt = p.tiles_per_seq - 1 - (w % p.tiles_per_seq);   // late (heavy) tiles first
    w /= p.tiles_per_seq;
    const int g = w % p.Hkv, b = w / p.Hkv;
    const Bounds sb = seq_bounds(p.cu_q, p.cu_k, b, p.total_q, p.total_k);
    const int tok0 = jt * p.T;
    if (tok0 >= sb.Sq) return;
    const int ntok = (sb.Sq - tok0) < p.T ? (sb.Sq - tok0) : p.T;
    const int off = sb.Sk - sb.Sq;
    // (max_seqlen_k bounds every S_k; a longer sequence is cut to it here)
    const int nb = p.nb_max;
    int nblk = (sb.Sk + kSelBlock - 1) / kSelBlock;
    nblk = nblk < nb ? nblk : nb;
    int ncmp = n_windows(sb.Sk);
    ncmp = ncmp < p.ncmp_max ? ncmp : p.ncmp_max;
    const int G = p.G;
    float* s_imp = reinterpret_cast<float*>(smem);                 // [T][nb]
    uint8_t* cbuf = smem + (((size_t)p.T * nb * 4 + 15) & ~(size_t)15);

    for (int x = tid; x < p.T * nb; x += kSelectThreads) s_imp[x] = 0.f;

    // this wave's m-tile: row = wave*16 + lr -> (token t_l, head hh)
    const int row = wave * 16 + lr;
    const int t_l = row / G, hh = row - t_l * G;
    const bool valid = wave < p.mtiles && t_l < ntok;
    const int c = tok0 + t_l + off;                    // the row's aligned key position
    int nvis = c >= kCmpSize - 1 ? (c - (kCmpSize - 1)) / kCmpStride + 1 : 0;
    nvis = nvis < ncmp ? nvis : ncmp;
    if (!valid) nvis = 0;
    // windows the tile's last token sees: the chunk count of every wave
    const int c_last = tok0 + ntok - 1 + off;
    int nv_tile = c_last >= kCmpSize - 1 ? (c_last - (kCmpSize - 1)) / kCmpStride + 1 : 0;
    nv_tile = nv_tile < ncmp ? nv_tile : ncmp;
    const int nch = (nv_tile + kWinChunk - 1) / kWinChunk;

    u32x4_t qf[KS];
    {
        const uint16_t* qr = p.q + ((sb.q0 + tok0 + (valid ? t_l : 0)) * p.Hq + g * G + hh) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = valid ? *reinterpret_cast<const u32x4_t*>(qr + s * 32 + lg * 8) : u32x4_t{0u, 0u, 0u, 0u};
    }
    const uint16_t* cbase = p.cmp + ((int64_t)b * p.ncmp_max * p.Hkv + g) * D;
    const int64_t cstride = (int64_t)p.Hkv * D;        // elements between windows
    const float c2 = p.scale_log2;

    // chunk staging: piece x = tid + 256 n -> window x / CPR, 8-dim piece x % CPR
    u32x4_t stg[NL];
    auto fetch = [&](int ch) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int x = tid + n * kSelectThreads;
            int wi = ch * kWinChunk + x / CPR;
            wi = wi < p.ncmp_max ? wi : p.ncmp_max - 1;          // (masked below)
            stg[n] = *reinterpret_cast<const u32x4_t*>(cbase + wi * cstride + (x % CPR) * 8);
        }
    };
    auto stage = [&](int buf) {
        uint8_t* dst = cbuf + buf * kChunkBytes;
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            const int x = tid + n * kSelectThreads;
            const int wr = x / CPR, pc = x % CPR;                 // window in chunk, piece
            const int kt = wr / 16, s = pc / 4;
            const int l = (pc % 4) * 16 + wr % 16;                // fragment lane
            *reinterpret_cast<u32x4_t*>(dst + (kt * KS + s) * 1024 + l * 16) = stg[n];
        }
    };
    // S^T of chunk ch from buffer buf: st[kt][i] = window ch*64 + 16kt + 4lg + i (log2 units)
    auto scores = [&](int ch, int buf, f32x4_t (&st)[4]) {
        const uint8_t* src = cbuf + buf * kChunkBytes + lane * 16;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                st[kt] = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(src + (kt * KS + s) * 1024), qf[s], st[kt]);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int wi = ch * kWinChunk + kt * 16 + lg * 4 + i;
                st[kt][i] = wi < nvis ? st[kt][i] * c2 : -INFINITY;
            }
    };

    // Two passes over the chunks: row max and sum, then probabilities ->
    // block masses of token t_l.  Step st_i runs chunk st_i % nch from buffer
    // st_i & 1 while the next step's chunk is fetched.
    float m = -INFINITY, l = 0.f, inv = 0.f;
    float* imp_row = s_imp + (valid ? t_l : 0) * nb;
    // lanes summed before an atomic: a token's rows within the m-tile (G
    // dividing 16), all 16 rows (G a multiple of 16), else none
    const int gsum = (16 % G == 0) ? G : (G % 16 == 0 ? 16 : 1);
    const int nsteps = 2 * nch;
    if (nsteps > 0) {
        fetch(0);
        stage(0);
    }
    __syncthreads();                                   // table cleared, chunk 0 staged
    for (int si = 0; si < nsteps; ++si) {
        const int ch = si % nch, buf = si & 1;
        if (si + 1 < nsteps) fetch((si + 1) % nch);
        f32x4_t st[4];
        if (wave < p.mtiles) {
            scores(ch, buf, st);
            if (si < nch) {                                         // pass 1
                float mx = m;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[kt][i]);
                if (mx != -INFINITY) {
                    float sum = 0.f;
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sum += fast_exp2(st[kt][i] - mx);
                    l = l * fast_exp2(m - mx) + sum;
                    m = mx;
                }
                if (si == nch - 1) {                                // the row's four lanes
#pragma unroll
                    for (int o = 16; o < 64; o <<= 1) {
                        const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
                        const float mn = fmaxf(m, mo);
                        if (mn != -INFINITY) {
                            l = (m == -INFINITY ? 0.f : l * fast_exp2(m - mn)) +
                                (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mn));
                            m = mn;
                        }
                    }
                    inv = l > 0.f ? 1.f / l : 0.f;
                }
            } else {                                                // pass 2
                // the rows of one token (its G heads) are adjacent lanes: their
                // masses are summed in registers first, and one lane per token
                // and block adds them to the table
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    float pr[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = st[kt][i] == -INFINITY ? 0.f : fast_exp2(st[kt][i] - m) * inv;
                    const int blk = ch * (kWinChunk / 4) + kt * 4 + lg;   // block of windows 4blk .. 4blk+3
                    const float own = group_sum(pr[0] + pr[1] + pr[2] + 0.5f * pr[3], gsum);
                    const float nxt = group_sum(0.5f * pr[3], gsum);
                    if (valid && (lr % gsum) == 0) {
                        if (own != 0.f) atomicAdd(imp_row + blk, own);
                        if (nxt != 0.f) atomicAdd(imp_row + blk + 1, nxt);
                    }
                }
            }
        }
        if (si + 1 < nsteps) stage((si + 1) & 1);
        __syncthreads();
    }

    // selection, when a token has at most 16 * kPickRegs candidates: four
    // tokens per wave, one per 16-lane row.  Each lane keeps its candidates
    // x = lo + (lane % 16) + 16 j in registers and every pick is a row-wide
    // argmax (DPP within the row), so a pick costs no LDS round trip.
    if (nblk - p.init <= 16 * kPickRegs) {
        const int grp = lane >> 4, l16 = lane & 15;
        for (int tb = 4 * wave; tb < ntok; tb += 4 * kSelectWaves) {
            const int t = tb + grp;
            const bool tv = t < ntok;
            const int ct = tok0 + t + off;
            int n = 0;
            int pick[4] = {-1, -1, -1, -1};             // entry l16 + 16 s of the list
            auto put = [&](int x) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    if (n == l16 + 16 * s4) pick[s4] = x;
                ++n;
            };
            int lo = 0, hi = 0;
            if (tv && ct >= 0) {
                const int qb = ct / kSelBlock < nblk - 1 ? ct / kSelBlock : nblk - 1;
                for (int x = 0; x < p.init && x <= qb && n < p.topk; ++x) put(x);
                for (int y = 0; y < p.local && n < p.topk; ++y) {
                    const int x = qb - y;
                    if (x < 0) break;
                    if (x >= p.init) put(x);            // (smaller ones are listed already)
                }
                lo = p.init;
                hi = qb - p.local + 1;
            }
            const float* imp = s_imp + (tv ? t : 0) * nb;
            float v[kPickRegs];
#pragma unroll
            for (int j = 0; j < kPickRegs; ++j) {
                const int x = lo + l16 + 16 * j;
                v[j] = x < hi ? imp[x] : -1.f;
            }
            bool go = n < p.topk && lo < hi;
            while (__builtin_amdgcn_ballot_w64(go) != 0ull) {
                unsigned long long key = 0ull;
#pragma unroll
                for (int j = 0; j < kPickRegs; ++j) {
                    const unsigned long long kj =
                        v[j] >= 0.f ? ((unsigned long long)__float_as_uint(v[j]) << 32) |
                                          (0xFFFFFFFFu - (uint32_t)(lo + l16 + 16 * j))
                                    : 0ull;
                    key = kj > key ? kj : key;
                }
                key = row_max_u64(key);
                if (go) {
                    if (key == 0ull) {
                        go = false;                     // no candidate left
                    } else {
                        const int x = (int)(0xFFFFFFFFu - (uint32_t)key);
                        put(x);
                        const int r = x - lo;
#pragma unroll
                        for (int j = 0; j < kPickRegs; ++j)
                            if (l16 == (r & 15) && j == (r >> 4)) v[j] = -1.f;   // used
                        go = n < p.topk;
                    }
                }
            }
            if (tv) {
                int32_t* out = p.blk_idx + ((sb.q0 + tok0 + t) * p.Hkv + g) * (int64_t)p.topk;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int e = l16 + 16 * s4;
                    if (e < p.topk) out[e] = e < n ? pick[s4] : -1;
                }
            }
        }
        return;
    }

    // selection otherwise: one wave per token
    for (int t = wave; t < ntok; t += kSelectWaves) {
        int32_t* out = p.blk_idx + ((sb.q0 + tok0 + t) * p.Hkv + g) * (int64_t)p.topk;
        const int ct = tok0 + t + off;
        int n = 0;
        int first = -1;                                 // this lane's pick, lane e holds entry e
        if (ct >= 0) {
            const int qb = ct / kSelBlock < nblk - 1 ? ct / kSelBlock : nblk - 1;
            for (int x = 0; x < p.init && x <= qb && n < p.topk; ++x) {
                if (lane == n) first = x;
                ++n;
            }
            for (int y = 0; y < p.local && n < p.topk; ++y) {
                const int x = qb - y;
                if (x < 0) break;
                if (x < p.init) continue;                   // already listed
                if (lane == n) first = x;
                ++n;
            }
            float* imp = s_imp + t * nb;
            const int lo = p.init, hi = qb - p.local + 1;
            while (n < p.topk && lo < hi) {
                unsigned long long best = 0ull;
                for (int x = lo + lane; x < hi; x += 64) {
                    const float v = imp[x];
                    if (v >= 0.f) {
                        const unsigned long long key =
                            ((unsigned long long)__float_as_uint(v) << 32) | (0xFFFFFFFFu - (uint32_t)x);
                        best = key > best ? key : best;
                    }
                }
                best = wave_max_u64(best);
                if (best == 0ull) break;                    // no candidate left
                const int x = (int)(0xFFFFFFFFu - (uint32_t)best);
                if (lane == n) first = x;
                if (lane == ((x - lo) & 63)) imp[x] = -1.f;  // used
                __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the mark lands first
                __builtin_amdgcn_wave_barrier();
                ++n;
            }
        }
        if (lane < p.topk) out[lane] = lane < n ? first : -1;   // (topk <= 64)
    }
}

size_t block_select_lds_bytes(int T, int nb_max, int D) {
    return (((size_t)T * nb_max * 4 + 15) & ~(size_t)15) + 2 * (size_t)kWinChunk * D * 2;
}

hipError_t launch_block_select(const BlockSelectParams& p, int D, hipStream_t stream) {
    const int64_t ncmp_items = (int64_t)p.batch * p.ncmp_max * p.Hkv * (D / 8);
    if (ncmp_items > 0) {
        const unsigned gc = (unsigned)((ncmp_items + 255) / 256);
        if (D == 64) hipLaunchKernelGGL(cmp_keys_kernel<64>, dim3(gc), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(cmp_keys_kernel<128>, dim3(gc), dim3(256), 0, stream, p);
    }
    const size_t lds = block_select_lds_bytes(p.T, p.nb_max, D);
    static bool attr_set[2] = {false, false};
    const int di = D == 64 ? 0 : 1;
    if (!attr_set[di]) {
        const void* f = D == 64 ? reinterpret_cast<const void*>(&block_select_kernel<64>)
                                : reinterpret_cast<const void*>(&block_select_kernel<128>);
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set[di] = true;
    }
    const unsigned grid = (unsigned)(p.batch * p.Hkv * p.tiles_per_seq);
    if (grid > 0) {
        if (D == 64) hipLaunchKernelGGL(block_select_kernel<64>, dim3(grid), dim3(kSelectThreads), lds, stream, p);
        else hipLaunchKernelGGL(block_select_kernel<128>, dim3(grid), dim3(kSelectThreads), lds, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fsa
