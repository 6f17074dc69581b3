// k1_project.hip -- LayerNorm_in fused into the gated input projection.
//
// For each pair (r, s) of a batch element:  x = LayerNorm_in(z_rs);
//   a_c = m_rs * (p_in x)_c     * sg((g_in x)_c),
//   b_c = m_rs * (p_in x)_(C+c) * sg((g_in x)_(C+c)),
// stored channel-major so that the contraction reads k-contiguous rows:
//   outgoing: pair (r, s) = (i, k) lands at row r, position s of channel c
//   incoming: pair (r, s) = (k, i) lands at row s, position r of channel c
// (the single-GPU form of the layout change the fold-cp-ops README performs
// between its two GEMMs).  fp32 rows are plain ([c][row][k]); bf16 rows are
// K-blocked ([c][k / 32][row][k % 32], kblk_off).
//
// Work split: a 256-thread workgroup is 4 waves; each wave owns ROWS pairs
// that are consecutive in the channel-major order (outgoing: consecutive s of
// one r; incoming: consecutive r of one s).  A wave loads its pairs' z rows
// straight into MFMA operand registers (lane l: pair l % 16 of a 16-row block,
// chunk l / 16 of each K-group), computes the LayerNorm statistics in fp32 with
// two cross-lane reductions, normalises in registers and keeps x as the A
// operand for the whole projection.  The projection weights stream through
// double-buffered LDS 64 rows at a time; each 64-row stage is (p rows, g rows)
// of 16 channels, twice, so the epilogue finds p and g of one channel in one
// lane.  Each lane's four results are four consecutive pairs of one channel,
// written as one 4-element run.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

template <typename T, int D>
struct K1Cfg {
    static constexpr int CE = Elem<T>::CE;
    static constexpr int RB = (sizeof(T) == 2) ? 4 : 2;   // 16-row blocks per wave
    static constexpr int ROWS = RB * 16;                   // pairs per wave
    static constexpr int DCH = D / CE;                     // chunks per z row
    static constexpr int KG = DCH / 4;                     // K-groups over D
    static constexpr int NCOL = 64;                        // weight rows per stage
    static constexpr int SWM = swz_mask(DCH);              // swizzle mask
    static constexpr int W_LD = NCOL * DCH / 256;          // chunks per thread per stage
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k1_project(
    const T* __restrict__ z, const T* __restrict__ mask, const T* __restrict__ W,
    const float* __restrict__ ln_w, const float* __restrict__ ln_b, float eps,
    T* __restrict__ a_cm, T* __restrict__ b_cm, int N, int C, int incoming, int blocks_per_b)
{
    using Cf = K1Cfg<T, D>;
    constexpr int CE = Cf::CE, RB = Cf::RB, ROWS = Cf::ROWS, DCH = Cf::DCH, KG = Cf::KG;
    constexpr int NCOL = Cf::NCOL, SWM = Cf::SWM, W_LD = Cf::W_LD;
    __shared__ u32x4 wlds[2][NCOL * DCH];
    __shared__ float s_w[D], s_b[D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t NN = (size_t)N * N;
    const int bidx = blockIdx.x / blocks_per_b;
    const int t = blockIdx.x % blocks_per_b;

    // Pair geometry of this wave: row m <-> pair index zpair(m) (natural r*N+s)
    // and channel-major position cm0 + m.  Rows >= mvalid do not exist.
    size_t zbase, zstride, cm0;
    int mvalid;
    if (!incoming) {
        size_t p0 = ((size_t)t * 4 + wave) * ROWS;
        zbase = p0; zstride = 1; cm0 = p0;
        mvalid = p0 < NN ? ROWS : 0;
    } else {
        const int rtiles = (N + ROWS - 1) / ROWS;
        const int rt = t % rtiles, st = t / rtiles;
        const int r0 = rt * ROWS, s = st * 4 + wave;
        zbase = (size_t)r0 * N + s; zstride = (size_t)N; cm0 = (size_t)s * N + r0;
        mvalid = min(ROWS, N - r0);
    }

    for (int d = tid; d < D; d += 256) { s_w[d] = ln_w[d]; s_b[d] = ln_b[d]; }

    // Offset within a channel slab of the four pairs this lane stores for
    // block rb (rows m0 .. m0 + 3 share a row of the slab: 4 divides N).
    constexpr DType TD = sizeof(T) == 2 ? DType::BF16 : DType::FP32;
    const size_t slab_ab = ab_slab_elems(TD, N);
    size_t spos[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const size_t pos = cm0 + rb * 16 + 4 * (lane >> 4);
        if constexpr (TD == DType::BF16) {
            const uint32_t row = (uint32_t)(pos / (size_t)N), k = (uint32_t)(pos - (size_t)row * N);
            spos[rb] = kblk_off(row, k, (uint32_t)N);
        } else {
            spos[rb] = pos;
        }
    }

    // Weight stage 0 in flight while z is loaded and normalised.
    u32x4 wr[W_LD];
    auto wload = [&](int q) {
#pragma unroll
        for (int it = 0; it < W_LD; ++it) {
            int idx = tid + 256 * it, row = idx / DCH, c = idx % DCH;
            wr[it] = ld16(W + ((size_t)(q * NCOL + row)) * D + c * CE);
        }
    };
    auto wstore = [&](int buf) {
#pragma unroll
        for (int it = 0; it < W_LD; ++it) {
            int idx = tid + 256 * it, row = idx / DCH, c = idx % DCH;
            wlds[buf][row * DCH + (c ^ (row & SWM))] = wr[it];
        }
    };
    wload(0);

    // x operand registers: block rb, K-group kg -> chunk kg*4 + lane/16 of row rb*16 + lane%16.
    u32x4 xf[RB][KG];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const T* zb = z + (size_t)bidx * NN * D;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = rb * 16 + (lane & 15);
        const T* zp = zb + (zbase + (size_t)m * zstride) * D;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
            xf[rb][kg] = (m < mvalid) ? ld16(zp + (kg * 4 + (lane >> 4)) * CE) : zero;
    }
    wstore(0);
    __syncthreads();  // s_w/s_b and weight stage 0 visible

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float v[KG][CE];
        float s = 0.f;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            Elem<T>::unpack(xf[rb][kg], v[kg]);
#pragma unroll
            for (int e = 0; e < CE; ++e) s += v[kg][e];
        }
        const float mu = sum_row_lanes(s) * (1.0f / D);
        float q = 0.f;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int e = 0; e < CE; ++e) { float dlt = v[kg][e] - mu; q += dlt * dlt; }
        const float rstd = rsqrtf(sum_row_lanes(q) * (1.0f / D) + eps);
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const int d0 = (kg * 4 + (lane >> 4)) * CE;
            float y[CE];
#pragma unroll
            for (int e = 0; e < CE; ++e) y[e] = (v[kg][e] - mu) * rstd * s_w[d0 + e] + s_b[d0 + e];
            xf[rb][kg] = Elem<T>::pack(y);
        }
    }

    // Mask of the pairs this lane's results belong to: rows rb*16 + 4*(lane/16) + r.
    float mv[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = rb * 16 + 4 * (lane >> 4) + r;
            mv[rb][r] = (mask && m < mvalid)
                            ? Elem<T>::load1(mask, (size_t)bidx * NN + zbase + (size_t)m * zstride)
                            : 1.0f;
        }

    const int nq = C / 16;           // 64-row stages: C/32 for a, then C/32 for b
    const int qa = C / 32;
    for (int q = 0; q < nq; ++q) {
        const int buf = q & 1;
        if (q + 1 < nq) wload(q + 1);
        f32x4 acc[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const int c = kg * 4 + (lane >> 4);
            u32x4 fb[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int row = nb * 16 + (lane & 15);
                fb[nb] = wlds[buf][row * DCH + (c ^ (row & SWM))];
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[rb][nb] = Elem<T>::mma(xf[rb][kg], fb[nb], acc[rb][nb]);
        }
        // Epilogue: blocks (0,1) = (p, g) of channels g0..g0+15, (2,3) of g0+16..g0+31.
        T* dst = (q < qa) ? a_cm : b_cm;
        const int gq = (q < qa) ? q : q - qa;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ch = gq * 32 + h * 16 + (lane & 15);
            T* dc = dst + ((size_t)bidx * C + ch) * slab_ab;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int m0 = rb * 16 + 4 * (lane >> 4);
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = mv[rb][r] * acc[rb][2 * h][r] * sigmoidf_(acc[rb][2 * h + 1][r]);
                if (m0 < mvalid) Elem<T>::store4(dc, spos[rb], o);
            }
        }
        if (q + 1 < nq) wstore(buf ^ 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// bf16 path for D in {128, 256}: LayerNorm folded into the projection.
//
// With mu and rstd = 1 / sqrt(var + eps) of a z row, every projection output
// is  W (gamma (z - mu) rstd + beta) = W' x + T  with x = (z - mu) rstd, W' the
// weights with gamma folded in (bf16) and T = W beta (computed at create time
// in fp64, kept as the fp32 start vector (T, T, T, T) of each row).  For gate
// rows W' and T also carry the factor -log2(e).  Statistics take one pass
// with v_dot2_f32_bf16 over the raw bf16 z held in registers; z is then
// normalised in place (x rounded to bf16), and the MFMA multiplies W' with
// it, each accumulator starting at its row's T.  A stage ends with
// acc_p = p and acc_g = -log2(e) g, so the epilogue per output is
// a = m acc_p / (1 + 2^acc_g) (no m without a mask).
//
// A workgroup is 4 waves of 64 pairs; a wave's pairs are two adjacent rows of
// the K-blocked a and b times one 32-wide k block, so each channel's 64 results
// are one whole 128-byte line.  Two workgroups share a CU, so one's epilogue
// overlaps the other's MFMAs.  The weights stream through a 3-slot LDS ring by
// global->LDS DMA, one 32-row stage ((p, g) rows of 16 channels) at a time, two
// stages ahead; rows are 2D bytes with 16-byte chunk c of row r stored at
// c ^ (r % 16).  A stage's results go through a per-wave LDS tile and leave as
// 16-byte stores of whole lines; lanes of pairs past the end store to a sink
// so that every wave issues the same number of stores per stage (the DMA
// waits count them).
// ---------------------------------------------------------------------------
namespace k1f {
constexpr int RB = 4, ROWS = RB * 16, NWV = 4, NSW = 3, CMAX = 256;
template <int D>
struct Cfg {
    static constexpr int KG = D / 32;
    static constexpr int STAGE = 32 * D * 2;                  // bytes per weight stage
    static constexpr int DPW = STAGE / 1024 / NWV;             // DMA instructions per wave per stage
    static constexpr int EXT = 4 * CMAX * 16;                  // accumulator start vectors
    static constexpr int SC = NWV * RB * 16 * 4;               // per-pair mask values
    static constexpr int OT = NWV * 16 * ROWS * 2;             // per-wave output tiles
    static constexpr int LDS = NSW * STAGE + EXT + SC + OT;
    static_assert(D == 128 || D == 256, "widths");
    static_assert(STAGE % (1024 * NWV) == 0, "DMA split");
};
}  // namespace k1f

// MK: a pair mask is given (every output is multiplied by its pair's mask
// value, zero for pairs past N).  Without one, outputs of pairs past N are
// not stored at all (their lanes write to the sink), so no multiply is needed.
template <int D, bool MK>
__global__ __launch_bounds__(256, 2) void k1_project_fold(
    const bf16* __restrict__ z, const bf16* __restrict__ mask, const bf16* __restrict__ Wf,
    const float* __restrict__ Tv, float eps, bf16* __restrict__ a_cm, bf16* __restrict__ b_cm,
    bf16* __restrict__ sink, int N, int C, int incoming, int blocks_per_b)
{
    using namespace k1f;
    using Cf = Cfg<D>;
    constexpr int KG = Cf::KG, STAGE = Cf::STAGE, DPW = Cf::DPW;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cf::LDS];
    unsigned char* ring = smem;
    f32x4* ext = reinterpret_cast<f32x4*>(smem + NSW * STAGE);
    float* sc = reinterpret_cast<float*>(smem + NSW * STAGE + Cf::EXT);
    // This wave's output tile of one stage: 16 channel rows of 64 pairs (128
    // bytes).  The 8-byte slot c of row r sits at c ^ (2 (r / 2)), so the
    // epilogue's 8-byte writes (lanes = 16 rows x 2 slots per 32 lanes) and the
    // 16-byte read-back (lanes = 2 rows x 8 chunks per 16 lanes) hit distinct
    // banks.
    unsigned char* otile = smem + NSW * STAGE + Cf::EXT + Cf::SC + (threadIdx.x >> 6) * 16 * ROWS * 2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t NN = (size_t)N * N;
    const int bidx = blockIdx.x / blocks_per_b;
    const int t = blockIdx.x % blocks_per_b;
    const int NQ = C / 8;   // stages: C/16 channel groups of a, then of b

    // Pair geometry.  A wave owns 64 pairs that fill whole 128-byte lines of
    // the K-blocked a and b: storage rows row0 and row0 + 1 (row0 even) times
    // the 32-wide k block [k0, k0 + 32).  MFMA row m is the pair at storage row
    // row0 + m / 32, k = k0 + m % 32; pairs with k >= N do not exist (only k
    // below k0 + kvalid does).
    //   outgoing: storage row i = z row, k = z column: z pair (row, k)
    //   incoming: storage row i = z column, k = z row: z pair (k, row)
    const int nkb = (N + 31) / 32;
    const int unit = t * NWV + wave;
    // Consecutive units take consecutive row pairs of one k block, so the
    // lines the workgroups in flight store are one contiguous run per channel
    // (measured 1-7 % faster than walking the k blocks of a row pair first).
    const int npr = N / 2;
    const int row0 = 2 * (unit % npr), k0 = 32 * (unit / npr);
    const int kvalid = unit < npr * nkb ? min(32, N - k0) : 0;   // the last workgroup may hold idle waves
    auto zpair = [&](int m) -> size_t {
        const size_t row = (size_t)(row0 + (m >> 5)), k = (size_t)(k0 + (m & 31));
        return incoming ? k * N + row : row * N + k;
    };

    // Per-lane source offsets (elements) of this wave's DMA instructions within
    // a stage: instruction qi = wave + 4 i fills bytes [qi KB, qi KB + 1 KB) of
    // the slot, i.e. row r = 1024 qi / 2D + l / (2D / 16), physical chunk
    // l % (2D / 16), holding logical chunk (physical ^ (r % 16)).  Row r grows
    // by 2048 i / D, a multiple of 8, so offsets of instruction i are those of
    // instruction i % 2 plus 16 (i / 2) rows.
    uint32_t doff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int qi = wave + i * NWV;
        const int byte = qi * 1024 + lane * 16;
        const int row = byte / (2 * D), pch = (byte % (2 * D)) / 16;
        doff[i] = (uint32_t)(row * D + (pch ^ (row & 15)) * 8);
    }
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_ring = lds_addr_of(ring);
    auto issue = [&](int q, const unsigned char* sl) {
        const bf16* w0 = Wf + (size_t)q * 32 * D;
        const uint32_t la = lds_ring + (uint32_t)(sl - ring) + (uint32_t)(wave_s * 1024);
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            dma16_to_lds(w0 + (i >> 1) * 16 * D + doff[i & 1], la + (uint32_t)(i * NWV * 1024));
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue loads, all in flight together: the raw z rows (MFMA A operand:
    // block rb, K-group kg -> chunk kg*4 + g4 of pair rb*16 + l16) and the mask
    // into registers, then the accumulator start vectors and the first three
    // weight stages into LDS by DMA.  Lanes of pairs that do not exist read pair 0
    // and are zeroed afterwards, so no load sits behind a branch.
    u32x4 zf[RB][KG];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* zb = z + (size_t)bidx * NN * D;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = rb * 16 + l16;
        const bool live = (m & 31) < kvalid;
        const bf16* zp = zb + (live ? zpair(m) : 0) * D;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const u32x4 v = ld16(zp + (kg * 4 + g4) * 8);
            zf[rb][kg] = live ? v : zero;
        }
    }
    float mval[RB];
    if constexpr (MK) {
        const bf16* mb = mask + (size_t)bidx * NN;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int m = rb * 16 + l16;
            const bool live = (m & 31) < kvalid;
            const float mv = (float)mb[live ? zpair(m) : 0];
            mval[rb] = live ? mv : 0.0f;
        }
    }
    {
        // Accumulator start vectors: 4C entries of 16 bytes, C/16 kilobytes.
        const uint32_t lds_ext = lds_addr_of(ext);
        for (int q = wave_s; q < C / 16; q += NWV)
            dma16_to_lds(Tv + (size_t)q * 256 + lane * 4, lds_ext + (uint32_t)(q * 1024));
    }
    // Older than the DMA of stages 1 and 2, so the prologue's wait for stage 0
    // covers every load above.
    issue(0, ring);
    issue(1, ring + STAGE);
    issue(2, ring + 2 * STAGE);   // NQ = C / 8 >= 4
    // Statistics (one v_dot2 pass over the raw bf16 row), then z is normalised
    // in place: each lane's registers hold (z - mu) rstd of its pair rows as
    // bf16 (RNE), the MFMA A operand.  Missing pairs hold zeros and stay zero.
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t w = zf[rb][kg][h];   // scalar copy before the bit cast
                const bf16x2 x = __builtin_bit_cast(bf16x2, w);
                s1 = __builtin_amdgcn_fdot2_f32_bf16(x, one2, s1, false);
                s2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, s2, false);
            }
        s1 = sum_row_lanes(s1);
        s2 = sum_row_lanes(s2);
        const float mu = s1 * (1.0f / D);
        const float ve = fmaxf(s2 * (1.0f / D) - mu * mu, 0.f) + eps;
        const float rstd = rsqrtf(ve);
        const float nmr = -mu * rstd;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t w = zf[rb][kg][h];
                const bf16x2 x = {(__bf16)fmaf(__uint_as_float(w << 16), rstd, nmr),
                                  (__bf16)fmaf(__uint_as_float(w & 0xffff0000u), rstd, nmr)};
                zf[rb][kg][h] = __builtin_bit_cast(uint32_t, x);
            }
        if (MK && g4 == 0) sc[(wave * RB + rb) * 16 + l16] = mval[rb];
    }
    // Stage 0 landed (at most the DMA of stages 1 and 2 may be outstanding),
    // then publish it, the start vectors and the mask values.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(2 * DPW));
    barrier();

    // Weight fragment (B operand) of K-group kg for row l16 of half hf (p or g):
    // chunk (kg*4 + g4) ^ l16 of row hf*16 + l16.
    int wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[j] = l16 * (2 * D) + ((g4 ^ (l16 & 3)) * 16) + ((j ^ (l16 >> 2)) << 6);
    auto wfrag = [&](const unsigned char* sl, int hf, int kg) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(sl + hf * 32 * D + wb[kg & 3] + 256 * (kg >> 2));
    };

    const bool full = kvalid == 32;   // wave-uniform: no tail lanes
    // Each stage runs in two halves of HB = RB / 2 pair blocks; a half is KG
    // steps, one per K-group.  Step s issues the LDS reads of step s + 2, the
    // half's 2 HB MFMAs of step s and a share of the previous half's epilogue,
    // so the sigmoid math is spread over the matrix-core work.  The last two
    // steps of a stage's first half prefetch the second half's first
    // fragments (same slot); the first half of a stage reads its own after the
    // barrier that publishes the stage.
    constexpr int HB = RB / 2;
    constexpr int NOUT = HB * 4;   // epilogue outputs per lane per half
    // Mask values of this lane's four output pairs in every block (they do not
    // change from stage to stage), two bf16 per register: the mask is bf16, so
    // the packing is exact, and each value is unpacked to fp32 by one shift or
    // mask where it is used.  Held as fp32 they cost 8 more registers, which
    // at D = 128 is one workgroup per CU fewer and at D = 256 spills.
    u32x2 mrr[RB];
    if constexpr (MK) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f32x4 mv = *reinterpret_cast<const f32x4*>(sc + (wave * RB + rb) * 16 + 4 * g4);
            mrr[rb] = u32x2{(__float_as_uint(mv[0]) >> 16) | (__float_as_uint(mv[1]) & 0xffff0000u),
                            (__float_as_uint(mv[2]) >> 16) | (__float_as_uint(mv[3]) & 0xffff0000u)};
        }
    }
    // Start vectors of this lane's output channel (column l16 of stage q's 16 p
    // rows and 16 g rows): every accumulator of a stage starts at its channel's
    // beta term, (T_p) x 4 and (-log2(e) T_g) x 4 (the gate rows of the folded
    // weights carry the factor -log2(e) as well).
    auto tvecs = [&](int q, f32x4& tp4, f32x4& tg4) {
        tp4 = ext[q * 32 + l16];
        tg4 = ext[q * 32 + 16 + l16];
    };
    auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
    // One epilogue output (index k of NOUT) of the half Hp whose accumulators
    // are pp = p and gp = -log2(e) g: a = m p / (1 + 2^gp); writes a block's
    // four pairs to the output tile after its fourth output.
    const int oswz = 2 * (l16 >> 1);
    auto epi_out = [&](auto hpc, int k, const f32x4* pp, const f32x4* gp, f32x4* ov) {
        constexpr int HP = decltype(hpc)::value;
        const int j = k / 4, e = k % 4, rb = HP * HB + j;
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gp[j][e]));
        if constexpr (MK) {
            const uint32_t w = mrr[rb][e >> 1];
            const float mv = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            ov[j][e] = mv * pp[j][e] * sg;
        }
        else ov[j][e] = pp[j][e] * sg;
        if (e == 3) {
            bf16x4 h;
            h[0] = (bf16)ov[j][0]; h[1] = (bf16)ov[j][1]; h[2] = (bf16)ov[j][2]; h[3] = (bf16)ov[j][3];
            *reinterpret_cast<bf16x4*>(otile + l16 * 128 + (((rb * 4 + g4) ^ oswz) << 3)) = h;
        }
    };
    // Store stage q's output tile: lane L reads the 16 bytes of pairs 8 (L % 8)
    // .. +7 of channel row L / 8 (+ 8 for the second instruction) and writes
    // them to the channel-major output, whole 128-byte runs per row.  Runs past
    // the end go to the sink, so every wave issues exactly two stores.
    // A channel's 64 pairs are one 128-byte line of the K-blocked storage
    // (rows row0, row0 + 1 of block k0 / 32), in MFMA row order.
    const int orow = lane >> 3, ochk = lane & 7;
    const size_t slab_ab = ab_slab_elems(DType::BF16, N);
    const uint32_t spos = kblk_off((uint32_t)row0, (uint32_t)k0, (uint32_t)N) + 8 * ochk;
    const bool olive = 8 * (ochk & 3) < kvalid;
    auto store_tile = [&](int q) {
        const int part = q < NQ / 2 ? 0 : 1;
        bf16* base = (part ? b_cm : a_cm) + ((size_t)bidx * C + (q - part * (NQ / 2)) * 16) * slab_ab + spos;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = orow + 8 * i;
            const u32x4 v = *reinterpret_cast<const u32x4*>(otile + r * 128 + (((2 * ochk) ^ (2 * (r >> 1))) << 3));
            bf16* p = (full || olive) ? base + (size_t)r * slab_ab : sink + lane * 8;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));   // streamed out, read back by K2 from HBM
        }
    };
    // One half: MFMAs of blocks H of stage qo (in slot sl) into ap/ag.  The B
    // operands (p and g weight fragments) are read two steps ahead: bq holds
    // those of the half's first two steps (second half: prefetched by the
    // first, which leaves them there).  If EPI, the previous half (HP,
    // accumulators pp/gp) is finished alongside.
    auto half = [&](auto hc, auto epic, auto hpc, const unsigned char* sl, u32x4 (&bq)[2][2], f32x4* ap,
                    f32x4* ag, int qo, const f32x4* pp, const f32x4* gp) {
        constexpr int H = decltype(hc)::value;
        constexpr bool EPI = decltype(epic)::value;
        static_assert(KG >= 2, "two-step operand pipeline");
        f32x4 ov[HB];
        f32x4 tp4, tg4;
        tvecs(qo, tp4, tg4);
        if (H == 0) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                bq[s2][0] = wfrag(sl, 0, s2);
                bq[s2][1] = wfrag(sl, 1, s2);
            }
        }
        u32x4 b0 = bq[0][0], b1 = bq[0][1], c0 = bq[1][0], c1 = bq[1][1];
#pragma unroll
        for (int st = 0; st < KG; ++st) {
            // Prefetch the B operands of step st + 2 (past the end of the first
            // half: the second half's first two steps, same slot).
            const bool pre = st + 2 < KG || H == 0;
            const int kn = st + 2 < KG ? st + 2 : st + 2 - KG;
            u32x4 n0, n1;
            if (pre) {
                n0 = wfrag(sl, 0, kn);
                n1 = wfrag(sl, 1, kn);
            }
            // This step's MFMAs, each followed by a share of the epilogue.
            const int lo = st * NOUT / KG, hi = (st + 1) * NOUT / KG;   // constants after unrolling
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                const u32x4 a = zf[H * HB + j][st];
                if (st == 0) {
                    ap[j] = Elem<bf16>::mma(a, b0, tp4);
                    ag[j] = Elem<bf16>::mma(a, b1, tg4);
                } else {
                    ap[j] = Elem<bf16>::mma(a, b0, ap[j]);
                    ag[j] = Elem<bf16>::mma(a, b1, ag[j]);
                }
            }
            if (EPI) {
#pragma unroll
                for (int k = lo; k < hi; ++k) epi_out(hpc, k, pp, gp, ov);
            }
            // Each step is a scheduling region of its own; within it the
            // compiler orders the MFMAs, the prefetch reads and the epilogue
            // arithmetic (measured 2-3 % faster than pinning one MFMA per three
            // VALU operations, and the same as grouping a half's whole epilogue
            // into its first or last step).
            fence();
            b0 = c0;
            b1 = c1;
            if (pre) { c0 = n0; c1 = n1; }
        }
        if (H == 0) {
            bq[0][0] = b0;
            bq[0][1] = b1;
            bq[1][0] = c0;
            bq[1][1] = c1;
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    f32x4 pA[HB], gA[HB], pB[HB], gB[HB];
    u32x4 bq[2][2];
    half(I0{}, F_{}, I1{}, ring, bq, pA, gA, 0, pB, gB);
    // One iteration of the stage loop: the second half of stage q (ring slot
    // S = q % NSW) and the first half of stage q + 1.  S is a constant in each
    // of the NSW unrolled copies, so every LDS address of an iteration is a
    // loop-invariant register plus an immediate offset.  Returns true after
    // the last stage's second half has been issued.
    static_assert(NSW == 3, "the stage loop is unrolled by the ring depth");
    auto iteration = [&](auto sc, int q) -> bool {
        constexpr int S = decltype(sc)::value;
        const unsigned char* sl = ring + S * STAGE;
        half(I1{}, T_{}, I0{}, sl, bq, pB, gB, q, pA, gA);   // second half of stage q
        if (q + 1 == NQ) return true;
        // Stage q + 1 must have landed.  Every wave issues, in this order per
        // iteration: the DMA of stage q + 3 (DPW instructions, while q + 3 <
        // NQ) and the two stores of stage q.  Stage q + 1's DMA was issued in
        // the prologue (q < 2) or two iterations back, so the operations newer
        // than it are: stage 2's DMA (q = 0); then stage q + 2's DMA and two
        // iterations' stores (DPW + 4), of which all but the last DPW + 2 may
        // be waited for; 4 stores when no DMA was issued in between.
        if (q == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(DPW));
        else if (q + 2 < NQ) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(DPW + 2));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(2));
        barrier();
        if (q + 3 < NQ) issue(q + 3, ring + S * STAGE);   // into the slot stage q used
        half(I0{}, T_{}, I1{}, ring + ((S + 1) % NSW) * STAGE, bq, pA, gA, q + 1, pB, gB);
        store_tile(q);                   // the tile is complete; stage q + 1's epilogue starts after
        return false;
    };
    for (int q = 0;; q += NSW) {
        if (iteration(std::integral_constant<int, 0>{}, q)) break;
        if (iteration(std::integral_constant<int, 1>{}, q + 1)) break;
        if (iteration(std::integral_constant<int, 2>{}, q + 2)) break;
    }
    {
        f32x4 ov[HB];
#pragma unroll
        for (int k = 0; k < NOUT; ++k) epi_out(I1{}, k, pB, gB, ov);
        store_tile(NQ - 1);
    }
}

template <typename T, int D>
static hipError_t launch_k1_t(const Params& p, const void* z, const void* mask, int B, int N,
                              int incoming, void* a, void* b, hipStream_t s)
{
    using Cf = K1Cfg<T, D>;
    int blocks_per_b;
    if (!incoming) {
        const size_t NN = (size_t)N * N;
        blocks_per_b = (int)((NN + 4 * Cf::ROWS - 1) / (4 * Cf::ROWS));
    } else {
        blocks_per_b = ((N + Cf::ROWS - 1) / Cf::ROWS) * (N / 4);
    }
    dim3 grid((unsigned)((size_t)B * blocks_per_b));
    hipLaunchKernelGGL((k1_project<T, D>), grid, dim3(256), 0, s, (const T*)z, (const T*)mask,
                       (const T*)p.w_proj, p.ln_in_w, p.ln_in_b, p.eps, (T*)a, (T*)b, N, p.C,
                       incoming, blocks_per_b);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_k1_d(const Params& p, const void* z, const void* mask, int B, int N,
                              int incoming, void* a, void* b, hipStream_t s)
{
    switch (p.D) {
    case 32: return launch_k1_t<T, 32>(p, z, mask, B, N, incoming, a, b, s);
    case 64: return launch_k1_t<T, 64>(p, z, mask, B, N, incoming, a, b, s);
    case 96: return launch_k1_t<T, 96>(p, z, mask, B, N, incoming, a, b, s);
    case 128: return launch_k1_t<T, 128>(p, z, mask, B, N, incoming, a, b, s);
    case 160: return launch_k1_t<T, 160>(p, z, mask, B, N, incoming, a, b, s);
    case 192: return launch_k1_t<T, 192>(p, z, mask, B, N, incoming, a, b, s);
    case 224: return launch_k1_t<T, 224>(p, z, mask, B, N, incoming, a, b, s);
    case 256: return launch_k1_t<T, 256>(p, z, mask, B, N, incoming, a, b, s);
    default: return hipErrorInvalidValue;
    }
}

bool project_supported(int D, int C, DType)
{
    return D >= 32 && D <= 256 && D % 32 == 0 && C >= 32 && C <= 256 && C % 32 == 0;
}

template <int D>
static hipError_t launch_k1_fold(const Params& p, const void* z, const void* mask, int B, int N,
                                 int incoming, void* a, void* b, hipStream_t s)
{
    using namespace k1f;
    const long long units = (long long)(N / 2) * ((N + 31) / 32);   // 64-pair units per batch element
    const int blocks_per_b = (int)((units + NWV - 1) / NWV);
    dim3 grid((unsigned)((size_t)B * blocks_per_b));
    if (mask)
        hipLaunchKernelGGL((k1_project_fold<D, true>), grid, dim3(256), 0, s, (const bf16*)z, (const bf16*)mask,
                           (const bf16*)p.w_proj_f, (const float*)p.x_proj, p.eps, (bf16*)a, (bf16*)b,
                           (bf16*)p.sink, N, p.C, incoming, blocks_per_b);
    else
        hipLaunchKernelGGL((k1_project_fold<D, false>), grid, dim3(256), 0, s, (const bf16*)z, nullptr,
                           (const bf16*)p.w_proj_f, (const float*)p.x_proj, p.eps, (bf16*)a, (bf16*)b,
                           (bf16*)p.sink, N, p.C, incoming, blocks_per_b);
    return hipGetLastError();
}

hipError_t launch_project(const Params& p, const Plan& plan, const void* z, const void* mask, int B, int N,
                          int incoming, void* a_cm, void* b_cm, hipStream_t s)
{
    (void)plan;
    if (p.dtype == DType::BF16 && p.D == 256)
        return launch_k1_fold<256>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    if (p.dtype == DType::BF16 && p.D == 128)
        return launch_k1_fold<128>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    if (p.dtype == DType::BF16) return launch_k1_d<bf16>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    return launch_k1_d<float>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
}

}  // namespace trimul
