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
constexpr int kOnePassChunks = 8;      // rows of at most this many chunks take the one-pass kernel
constexpr float kSelLazy = 8.f;        // the one-pass maximum moves when passed by more than this (log2)
constexpr float kSelFar = -1e30f;      // its start: finite, so 2^(-inf - m) is 0 without a test

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

// maximum (MAX) or sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four rows),
// every lane getting it: the gfx950 permlane16 and permlane32 swaps
template <bool MAX>
__device__ __forceinline__ float rows4_combine(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

// maximum of a 64-bit key over each 16-lane row (every lane of the row gets
// it): the row maximum of the high words, then of the low words of the lanes
// that hold it -- quad swaps, then the half-row and row mirrors, each step one
// max with a DPP operand
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
    return x;
}
__device__ __forceinline__ unsigned long long row_max_u64(unsigned long long x) {
    const uint32_t hi = row_max_u32((uint32_t)(x >> 32));
    const uint32_t lo = row_max_u32((uint32_t)(x >> 32) == hi ? (uint32_t)x : 0u);
    return ((unsigned long long)hi << 32) | lo;
}

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
// LDS: the importance table [T][row stride] fp32, then two buffers of one chunk
// of 64 window summaries in MFMA A-operand order -- fragment (kt, s), 1 KiB,
// lane l's 16 bytes = C[16kt + l%16][32s + 8(l/16) .. +8] -- so every operand
// read is one contiguous wave read.  The chunk is loaded once per workgroup
// (all waves share it), the next one while the current one is used.
// Six waves per SIMD (80 VGPRs): three workgroups share a CU, as the LDS
// allows; at the compiler's own choice of 92 VGPRs only two fit.
template <int D, int NCH>
__global__ void __launch_bounds__(kSelectThreads, NCH == 0 ? 6 : 4) block_select_kernel(const BlockSelectParams p) {
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
    const int nbs = select_row_stride(nb);
    float* s_imp = reinterpret_cast<float*>(smem);                 // [T][nbs]
    uint8_t* cbuf = smem + (((size_t)p.T * nbs * 4 + 15) & ~(size_t)15);

    for (int x = tid; x < p.T * nbs; x += kSelectThreads) s_imp[x] = 0.f;

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

    // chunk staging: piece y = tid + n * threads is lane y % 64 of fragment
    // f = y / 64 = (kt, s) = (f / KS, f % KS), i.e. window 16 kt + y % 16 of
    // the chunk, 8-dim piece 4 s + (y % 64) / 16; its LDS place is y * 16, so
    // each wave's store fills one whole fragment (no bank conflicts)
    u32x4_t stg[NL];
    auto piece_window = [&](int n) {
        const int y = tid + n * kSelectThreads;
        return 16 * ((y / 64) / KS) + (y & 15);
    };
    auto piece_dims = [&](int n) {                      // first of the piece's 8 dims
        const int y = tid + n * kSelectThreads;
        return 8 * (4 * ((y / 64) % KS) + ((y & 63) >> 4));
    };
    auto fetch = [&](int ch) {
#pragma unroll
        for (int n = 0; n < NL; ++n) {
            int wi = ch * kWinChunk + piece_window(n);
            wi = wi < p.ncmp_max ? wi : p.ncmp_max - 1;          // (masked below)
            stg[n] = *reinterpret_cast<const u32x4_t*>(cbase + wi * cstride + piece_dims(n));
        }
    };
    auto stage = [&](int buf) {
        uint8_t* dst = cbuf + buf * kChunkBytes;
#pragma unroll
        for (int n = 0; n < NL; ++n)
            *reinterpret_cast<u32x4_t*>(dst + (tid + n * kSelectThreads) * 16) = stg[n];
    };
    // S^T of the chunk in buffer buf: st[kt][i] = <q_row, c_w> for window
    // w = ch*64 + 16kt + 4lg + i of chunk ch
    auto products = [&](int buf, f32x4_t (&st)[4]) {
        const uint8_t* src = cbuf + buf * kChunkBytes + lane * 16;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                st[kt] = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(src + (kt * KS + s) * 1024), qf[s], st[kt]);
    };
    // windows the row does not see -> -inf
    auto mask = [&](int ch, f32x4_t (&st)[4]) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int wi = ch * kWinChunk + kt * 16 + lg * 4 + i;
                st[kt][i] = wi < nvis ? st[kt][i] : -INFINITY;
            }
    };

    float* imp_row = s_imp + (valid ? t_l : 0) * nbs;
    // lanes summed before an atomic: a token's rows within the m-tile (G
    // dividing 16), all 16 rows (G a multiple of 16), else none
    const int gsum = (16 % G == 0) ? G : (G % 16 == 0 ? 16 : 1);
    if constexpr (NCH == 0) {
    // Two passes over the chunks: row max and sum, then probabilities ->
    // block masses of token t_l.  Step st_i runs chunk st_i % nch from buffer
    // st_i & 1 while the next step's chunk is fetched (every step fetches and
    // stages one, the last step chunk 0 again, unused, so that the loads are
    // unconditional).  Scores stay raw; the scale folds into the exponent's
    // FMA, and chunks every row of the wave sees whole skip the mask.
    float m = -INFINITY, l = 0.f, inv = 0.f;
    const int nsteps = 2 * nch;
    // the wave's first row has its fewest visible windows
    const int nvis0 = __builtin_amdgcn_readfirstlane(nvis);
    if (nsteps > 0) {
        fetch(0);
        stage(0);
    }
    __syncthreads();                                   // table cleared, chunk 0 staged
    for (int si = 0; si < nsteps; ++si) {
        const int ch = si % nch, buf = si & 1;
        fetch((si + 1) % nch);
        f32x4_t st[4];
        if (wave < p.mtiles) {
            products(buf, st);
            if ((ch + 1) * kWinChunk > nvis0) mask(ch, st);
            if (si < nch) {                                         // pass 1
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[kt][i]);
                mx = fmaxf(m, mx * c2);                             // (c2 > 0; -inf stays -inf)
                if (mx != -INFINITY) {
                    float sum = 0.f;
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sum += fast_exp2(fmaf(st[kt][i], c2, -mx));
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
                    for (int i = 0; i < 4; ++i)
                        pr[i] = st[kt][i] == -INFINITY ? 0.f : fast_exp2(fmaf(st[kt][i], c2, -m)) * inv;
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
        stage((si + 1) & 1);
        __syncthreads();
    }
    } else {
    // One pass, for rows of at most NCH chunks.  A row's windows are spread
    // over its four lanes (lg); the four share a lazily moved maximum m (log2
    // units) that moves only when a chunk's row maximum passes it by more
    // than kSelLazy, every mass held so far being scaled by 2^(m_old - m_new)
    // then, so each exponential is at most 2^kSelLazy.  mass[ch][kt] of lane
    // (lr, lg) is the unnormalised mass of block b = ch*16 + kt*4 + lg: its
    // windows 4b .. 4b+2, half of 4b+3, and half of 4b-1, which the lane of
    // block b-1 (16 lanes down, the last row passing into the next key tile or
    // chunk) hands over.  The masses reach the table once, after the loop.
    float mass[NCH][4];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mass[c][kt] = 0.f;
    float carry = 0.f;                                 // lanes lg = 0: half of the last window so far
    float m = kSelFar, lsum = 0.f;
    // the wave's first row has its fewest visible windows: chunks it sees
    // whole need no mask
    const int nvis0 = __builtin_amdgcn_readfirstlane(nvis);
    const int down = ((lane + 48) & 63) << 2;          // ds_bpermute address of lane - 16
    const int nc = nch < NCH ? nch : NCH;              // (the launcher keeps nch <= NCH)
    // Chunk loads through a buffer resource over this sequence's windows: a
    // window past the last reads as zeros, so every load is issued without a
    // clamp or a condition (the chunk after the last is fetched and staged
    // unused), and the wait counts stay exact across iterations.
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)cbase, 0, p.ncmp_max > 0 ? (uint32_t)(((int64_t)p.ncmp_max - 1) * cstride * 2 + D * 2) : 0u,
        0x00020000);
    int voff[NL];                                      // this thread's bytes within a chunk
#pragma unroll
    for (int n = 0; n < NL; ++n) voff[n] = piece_window(n) * (int)cstride * 2 + piece_dims(n) * 2;
    const int chunk_bytes = kWinChunk * (int)cstride * 2;
    auto fetch1 = [&](int ch) {
#pragma unroll
        for (int n = 0; n < NL; ++n) stg[n] = __builtin_amdgcn_raw_buffer_load_b128(crs, voff[n], ch * chunk_bytes, 0);
    };
    if (nc > 0) {
        fetch1(0);
        stage(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): the q fragments are in
    __syncthreads();                                   // table cleared, chunk 0 staged
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch >= nc) break;
        {
            fetch1(ch + 1);
            if (wave < p.mtiles) {
                f32x4_t st[4];
                products(ch & 1, st);
                if ((ch + 1) * kWinChunk > nvis0) mask(ch, st);
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    mx = fmaxf(mx, fmaxf(fmaxf(st[kt][0], st[kt][1]), fmaxf(st[kt][2], st[kt][3])));
                mx = rows4_combine<true>(mx) * c2;     // (c2 > 0; -inf stays -inf)
                if (mx > m + kSelLazy) {
                    const float f = fast_exp2(m - mx);
#pragma unroll
                    for (int c = 0; c < ch; ++c)
#pragma unroll
                        for (int kt = 0; kt < 4; ++kt) mass[c][kt] *= f;
                    carry *= f;
                    lsum *= f;
                    m = mx;
                }
                float own[4], sh[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    float pr[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(fmaf(st[kt][i], c2, -m));
                    const float s3 = pr[0] + pr[1] + pr[2];
                    lsum += s3 + pr[3];
                    own[kt] = fmaf(0.5f, pr[3], s3);
                    sh[kt] = __int_as_float(__builtin_amdgcn_ds_bpermute(down, __float_as_int(0.5f * pr[3])));
                }
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    mass[ch][kt] = own[kt] + (lg > 0 ? sh[kt] : (kt > 0 ? sh[kt - 1] : carry));
                carry = sh[3];
            }
            stage((ch + 1) & 1);
            __syncthreads();
        }
    }
    if (wave < p.mtiles) {
        const float l = rows4_combine<false>(lsum);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const bool writer = valid && (lr % gsum) == 0;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            if (ch < nc) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const int blk = ch * (kWinChunk / 4) + kt * 4 + lg;
                    const float v = group_sum(mass[ch][kt] * inv, gsum);
                    if (writer && v != 0.f && blk < nb) atomicAdd(imp_row + blk, v);
                }
            }
        }
        const int blk = nc * (kWinChunk / 4);          // half of the last window, lanes lg = 0
        const float v = group_sum(carry * inv, gsum);
        if (writer && lg == 0 && v != 0.f && blk < nb) atomicAdd(imp_row + blk, v);
    }
    __syncthreads();
    }

    // selection, when a token has at most 16 * kPickRegs candidates: four
    // tokens per wave, one per 16-lane row.  Each lane sorts its candidates
    // x = lo + (lane % 16) + 16 j once; a pick is a row-wide maximum of the
    // lanes' first keys (DPP within the row), and the row's first lane stores
    // the entry to the output list at once.
    if (nblk - p.init <= 16 * kPickRegs) {
        const int grp = lane >> 4, l16 = lane & 15;
        // keys 2 .. 7 of each lane's sorted list, [6][threads], in the chunk
        // buffers (unused from here on)
        unsigned long long* s_key = reinterpret_cast<unsigned long long*>(cbuf);
        for (int tb = 4 * wave; tb < ntok; tb += 4 * kSelectWaves) {
            const int t = tb + grp;
            const bool tv = t < ntok;
            const int ct = tok0 + t + off;
            int32_t* out = p.blk_idx + ((sb.q0 + tok0 + (tv ? t : 0)) * p.Hkv + g) * (int64_t)p.topk;
            int n = 0;
            auto put = [&](int x) {
                if (l16 == 0) out[n] = x;
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
            // the lane's candidates as 64-bit keys (importance bits, then the
            // inverted id: the larger key is the larger importance, ties to
            // the smaller block; 0 = none), sorted once in descending order;
            // a pick is the row maximum of the lanes' first keys, and the
            // lane that holds it moves on to its next key
            const float* imp = s_imp + (tv ? t : 0) * nbs;
            unsigned long long key[kPickRegs];
#pragma unroll
            for (int j = 0; j < kPickRegs; ++j) {
                const int x = lo + l16 + 16 * j;
                key[j] = x < hi ? ((unsigned long long)__float_as_uint(imp[x]) << 32) | (0xFFFFFFFFu - (uint32_t)x)
                                : 0ull;
            }
            // Batcher's odd-even merge sort of eight keys (19 compare-exchanges)
            auto cx = [&](int a, int b) {
                const unsigned long long hi_ = key[a] > key[b] ? key[a] : key[b];
                const unsigned long long lo_ = key[a] > key[b] ? key[b] : key[a];
                key[a] = hi_;
                key[b] = lo_;
            };
            static_assert(kPickRegs == 8, "sorting network for eight keys");
            cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
            cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
            cx(1, 2); cx(5, 6);
            cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
            cx(2, 4); cx(3, 5);
            cx(1, 2); cx(3, 4); cx(5, 6);
#pragma unroll
            for (int j = 2; j < kPickRegs; ++j) s_key[(j - 2) * kSelectThreads + tid] = key[j];
            unsigned long long head = key[0], nxt = key[1];   // the lane's next two keys
            int h = 2;                                         // the one after them
            bool go = n < p.topk && lo < hi;
            while (__builtin_amdgcn_ballot_w64(go) != 0ull) {
                const unsigned long long best = row_max_u64(head);
                if (go) {
                    if (best == 0ull) {
                        go = false;                     // no candidate left
                    } else {
                        put((int)(0xFFFFFFFFu - (uint32_t)best));
                        if (head == best) {             // this lane's key: the next one comes up
                            head = nxt;
                            nxt = h < kPickRegs ? s_key[(h - 2) * kSelectThreads + tid] : 0ull;
                            ++h;
                        }
                        go = n < p.topk;
                    }
                }
            }
            if (tv) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int e = l16 + 16 * s4;
                    if (e < p.topk && e >= n) out[e] = -1;
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
            // lane l's candidates are x = lo + l + 64 j, as 64-bit keys
            // (importance bits, inverted id; 0 = none).  A lane keeps its
            // largest key k1 and, until k1 is first taken, its second k2; a
            // pick is the wave maximum of the k1s.  The lane that held it
            // moves k2 up the first time and otherwise scans its candidates
            // again for the largest key below the one just taken, so a scan
            // happens only for a lane's second and later picks.
            const float* imp = s_imp + t * nbs;
            const int lo = p.init, hi = qb - p.local + 1;
            auto key_of = [&](int x) {
                return ((unsigned long long)__float_as_uint(imp[x]) << 32) | (0xFFFFFFFFu - (uint32_t)x);
            };
            unsigned long long k1 = 0ull, k2 = 0ull;
            for (int x = lo + lane; x < hi; x += 64) {
                const unsigned long long key = key_of(x);
                k2 = key > k1 ? k1 : (key > k2 ? key : k2);
                k1 = key > k1 ? key : k1;
            }
            bool k2_held = true;
            while (n < p.topk && lo < hi) {
                const unsigned long long best = wave_max_u64(k1);
                if (best == 0ull) break;                    // no candidate left
                const int x = (int)(0xFFFFFFFFu - (uint32_t)best);
                if (lane == n) first = x;
                ++n;
                if (k1 == best) {                           // (keys are distinct)
                    if (k2_held) {
                        k1 = k2;
                        k2_held = false;
                    } else {
                        unsigned long long nb1 = 0ull;      // the largest key below best
                        for (int y = lo + lane; y < hi; y += 64) {
                            const unsigned long long key = key_of(y);
                            nb1 = key < best && key > nb1 ? key : nb1;
                        }
                        k1 = nb1;
                    }
                }
            }
        }
        if (lane < p.topk) out[lane] = lane < n ? first : -1;   // (topk <= 64)
    }
}

size_t block_select_lds_bytes(int T, int nb_max, int D) {
    // the chunk buffers, which then hold keys 2 .. kPickRegs-1 of each thread
    const size_t chunks = 2 * (size_t)kWinChunk * D * 2;
    const size_t keys = (size_t)(kPickRegs - 2) * kSelectThreads * 8;
    return (((size_t)T * select_row_stride(nb_max) * 4 + 15) & ~(size_t)15) + (chunks > keys ? chunks : keys);
}

hipError_t launch_block_select(const BlockSelectParams& p, int D, hipStream_t stream) {
    const int64_t ncmp_items = (int64_t)p.batch * p.ncmp_max * p.Hkv * (D / 8);
    if (ncmp_items > 0) {
        const unsigned gc = (unsigned)((ncmp_items + 255) / 256);
        if (D == 64) hipLaunchKernelGGL(cmp_keys_kernel<64>, dim3(gc), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(cmp_keys_kernel<128>, dim3(gc), dim3(256), 0, stream, p);
    }
    const size_t lds = block_select_lds_bytes(p.T, p.nb_max, D);
    // rows of at most kOnePassChunks chunks of windows: the one-pass kernel
    // (and 32-bit byte offsets over a sequence's windows)
    const bool one = (p.ncmp_max + kWinChunk - 1) / kWinChunk <= kOnePassChunks &&
                     (int64_t)(kOnePassChunks + 1) * kWinChunk * p.Hkv * D * 2 < (int64_t)1 << 31;
    static std::atomic<unsigned long long> lds_set[4];     // devices with the LDS limit raised
    const int di = (D == 64 ? 0 : 1) + (one ? 2 : 0);
    const void* f = D == 64 ? (one ? reinterpret_cast<const void*>(&block_select_kernel<64, kOnePassChunks>)
                                   : reinterpret_cast<const void*>(&block_select_kernel<64, 0>))
                            : (one ? reinterpret_cast<const void*>(&block_select_kernel<128, kOnePassChunks>)
                                   : reinterpret_cast<const void*>(&block_select_kernel<128, 0>));
    hipError_t e = ensure_lds_limit(f, lds_set[di]);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(p.batch * p.Hkv * p.tiles_per_seq);
    if (grid > 0) {
        const dim3 gd(grid), bd(kSelectThreads);
        if (D == 64) {
            if (one) hipLaunchKernelGGL((block_select_kernel<64, kOnePassChunks>), gd, bd, lds, stream, p);
            else hipLaunchKernelGGL((block_select_kernel<64, 0>), gd, bd, lds, stream, p);
        } else {
            if (one) hipLaunchKernelGGL((block_select_kernel<128, kOnePassChunks>), gd, bd, lds, stream, p);
            else hipLaunchKernelGGL((block_select_kernel<128, 0>), gd, bd, lds, stream, p);
        }
    }
    return hipGetLastError();
}

}  // namespace fsa
