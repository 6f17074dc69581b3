// k1_project.hip -- LayerNorm_in fused into the gated input projection.
//
// For each pair (r, s) of a batch element:  x = LayerNorm_in(z_rs);
//   a_c = m_rs * (p_in x)_c     * sg((g_in x)_c),
//   b_c = m_rs * (p_in x)_(C+c) * sg((g_in x)_(C+c)),
// stored channel-major so that the contraction reads k-contiguous rows:
//   outgoing: pair (r, s) = (i, k) lands at a_cm[c][r*N + s]
//   incoming: pair (r, s) = (k, i) lands at a_cm[c][s*N + r]
// (the single-GPU form of the layout change the fold-cp-ops README performs
// between its two GEMMs).
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
            T* dc = dst + ((size_t)bidx * C + ch) * NN + cm0;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int m0 = rb * 16 + 4 * (lane >> 4);
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = mv[rb][r] * acc[rb][2 * h][r] * sigmoidf_(acc[rb][2 * h + 1][r]);
                if (m0 < mvalid) Elem<T>::store4(dc, (size_t)m0, o);
            }
        }
        if (q + 1 < nq) wstore(buf ^ 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// bf16 path for D in {128, 256}: LayerNorm folded into the projection.
//
// With mu, rstd = 1 / sqrt(var + eps) and sd = 1 / rstd of a z row, every
// projection output is  W (gamma (z - mu) rstd + beta) = rstd (W' z - mu S + T sd)
// where W' is W with gamma folded in (bf16), S its row sums and T = W beta
// (both computed at create time, each split into bf16 high and low parts).
// The MFMA multiplies W' with the raw bf16 z held in registers; one extra
// K-group per block (lane group 0 holds -mu_h, -mu_h, -mu_l, sd_h, sd_h, sd_l
// against S_h, S_l, S_h, T_h, T_l, T_h) adds the rest, so no element of z is
// normalised explicitly.  Statistics take one pass with v_dot2_f32_bf16.
// Epilogue per output: a = (m rstd acc_p) / (1 + 2^(-log2(e) rstd acc_g)).
//
// A workgroup is 4 waves of 64 pairs (geometry as in k1_project); two
// workgroups share a CU, so one's epilogue overlaps the other's MFMAs.  The
// weights stream through a 3-slot LDS ring by global->LDS DMA, one 32-row stage
// ((p, g) rows of 16 channels) at a time, two stages ahead; rows are 2D bytes
// with 16-byte chunk c of row r stored at c ^ (r % 16).  Each lane's results
// are four consecutive pairs of one channel, stored as one 8-byte run; lanes
// of pairs past the end store to a sink so that every wave issues the same
// number of stores per stage (the DMA waits count them).
// ---------------------------------------------------------------------------
namespace k1f {
constexpr int RB = 4, ROWS = RB * 16, NWV = 4, NSW = 3, CMAX = 256;
constexpr float LOG2E = 1.4426950408889634f;
template <int D>
struct Cfg {
    static constexpr int KG = D / 32;
    static constexpr int STAGE = 32 * D * 2;                  // bytes per weight stage
    static constexpr int DPW = STAGE / 1024 / NWV;             // DMA instructions per wave per stage
    static constexpr int EXT = 4 * CMAX * 16;                  // correction rows
    static constexpr int SC = NWV * RB * 2 * 16 * 4;           // per-pair scales
    static constexpr int LDS = NSW * STAGE + EXT + SC;
    static_assert(D == 128 || D == 256, "widths");
    static_assert(STAGE % (1024 * NWV) == 0, "DMA split");
};
}  // namespace k1f

#define TRIMUL_K1_LDS3(p) ((__attribute__((address_space(3))) void*)(p))

template <int D>
__global__ __launch_bounds__(256, 2) void k1_project_fold(
    const bf16* __restrict__ z, const bf16* __restrict__ mask, const bf16* __restrict__ Wf,
    const bf16* __restrict__ Xf, float eps, bf16* __restrict__ a_cm, bf16* __restrict__ b_cm,
    bf16* __restrict__ sink, int N, int C, int incoming, int blocks_per_b)
{
    using namespace k1f;
    using Cf = Cfg<D>;
    constexpr int KG = Cf::KG, STAGE = Cf::STAGE, DPW = Cf::DPW;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cf::LDS];
    unsigned char* ring = smem;
    u32x4* ext = reinterpret_cast<u32x4*>(smem + NSW * STAGE);
    float* sc = reinterpret_cast<float*>(smem + NSW * STAGE + Cf::EXT);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t NN = (size_t)N * N;
    const int bidx = blockIdx.x / blocks_per_b;
    const int t = blockIdx.x % blocks_per_b;
    const int NQ = C / 8;   // stages: C/16 channel groups of a, then of b

    // Pair geometry: row m <-> z pair zbase + m * zstride, channel-major position cm0 + m.
    size_t zbase, zstride, cm0;
    int mvalid;
    if (!incoming) {
        const size_t p0 = ((size_t)t * NWV + wave) * ROWS;
        zbase = p0; zstride = 1; cm0 = p0;
        mvalid = p0 < NN ? (int)min((size_t)ROWS, NN - p0) : 0;
    } else {
        const int rtiles = (N + ROWS - 1) / ROWS;
        const int rt = t % rtiles, st = t / rtiles;
        const int r0 = rt * ROWS, s = st * NWV + wave;
        zbase = (size_t)r0 * N + s; zstride = (size_t)N; cm0 = (size_t)s * N + r0;
        mvalid = min(ROWS, N - r0);
    }

    auto issue = [&](int q) {
        const bf16* w0 = Wf + (size_t)q * 32 * D;
        unsigned char* sl = ring + (q % NSW) * STAGE;
        int ln = threadIdx.x & 63;   // opaque: keeps per-lane offsets out of loop-carried registers
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int qi = wave + i * NWV;
            const int byte = qi * 1024 + ln * 16;
            const int row = byte / (2 * D), pch = (byte % (2 * D)) / 16;
            const bf16* src = w0 + (size_t)row * D + (pch ^ (row & 15)) * 8;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             TRIMUL_K1_LDS3(sl + qi * 1024), 16, 0, 0);
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(0);
    issue(1);   // NQ = C / 8 >= 4
    for (int i = tid; i < 4 * C; i += 256) ext[i] = ld16(Xf + (size_t)i * 8);

    // Raw z rows as the MFMA A operand: block rb, K-group kg -> chunk kg*4 + g4
    // of pair rb*16 + l16.  K-group KG is the correction fragment.
    u32x4 zf[RB][KG + 1];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* zb = z + (size_t)bidx * NN * D;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = rb * 16 + l16;
        const bf16* zp = zb + (zbase + (size_t)m * zstride) * D;
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) zf[rb][kg] = (m < mvalid) ? ld16(zp + (kg * 4 + g4) * 8) : zero;
    }
    float mval[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = rb * 16 + l16;
        mval[rb] = m < mvalid ? (mask ? (float)mask[(size_t)bidx * NN + zbase + (size_t)m * zstride] : 1.0f)
                              : 0.0f;
    }
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
        const float sd = ve * rstd;
        const __bf16 nmh = (__bf16)(-mu), nml = (__bf16)(-mu - (float)nmh);
        const __bf16 sdh = (__bf16)sd, sdl = (__bf16)(sd - (float)sdh);
        const __bf16 zr = (__bf16)0.0f;
        bf16x8 f = {zr, zr, zr, zr, zr, zr, zr, zr};
        if (g4 == 0) f = bf16x8{nmh, nmh, nml, sdh, sdh, sdl, zr, zr};
        zf[rb][KG] = __builtin_bit_cast(u32x4, f);
        if (g4 == 0) {
            sc[((wave * RB + rb) * 2 + 0) * 16 + l16] = -rstd * LOG2E;
            sc[((wave * RB + rb) * 2 + 1) * 16 + l16] = mval[rb] * rstd;
        }
    }
    // Stage 0 landed (at most stage 1's DMA may be outstanding), then publish
    // it, the correction rows and the scales.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(DPW));
    barrier();

    // Weight fragment (B operand) of K-group kg for row l16 of half hf (p or g):
    // chunk (kg*4 + g4) ^ l16 of row hf*16 + l16.
    int wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[j] = l16 * (2 * D) + ((g4 ^ (l16 & 3)) * 16) + ((j ^ (l16 >> 2)) << 6);
    auto wfrag = [&](const unsigned char* sl, int hf, int kg) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(sl + hf * 32 * D + wb[kg & 3] + 256 * (kg >> 2));
    };

    for (int q = 0; q < NQ; ++q) {
        if (q + 2 < NQ) issue(q + 2);    // into the slot stage q - 1 used
        const unsigned char* sl = ring + (q % NSW) * STAGE;
        f32x4 ap[RB], ag[RB];
        {
            const u32x4 ep = g4 == 0 ? ext[q * 32 + l16] : zero;
            const u32x4 eg = g4 == 0 ? ext[q * 32 + 16 + l16] : zero;
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                ap[rb] = Elem<bf16>::mma(zf[rb][KG], ep, z4);
                ag[rb] = Elem<bf16>::mma(zf[rb][KG], eg, z4);
            }
        }
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
            const u32x4 wp = wfrag(sl, 0, kg), wg = wfrag(sl, 1, kg);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                ap[rb] = Elem<bf16>::mma(zf[rb][kg], wp, ap[rb]);
                ag[rb] = Elem<bf16>::mma(zf[rb][kg], wg, ag[rb]);
            }
        }
        // Lane holds channel l16 of the group, pairs rb*16 + 4*g4 + e.
        const int half = q < NQ / 2 ? 0 : 1;
        const int ch = (q - half * (NQ / 2)) * 16 + l16;
        bf16* dst = (half ? b_cm : a_cm) + ((size_t)bidx * C + ch) * NN + cm0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f32x4 cx = *reinterpret_cast<const f32x4*>(sc + ((wave * RB + rb) * 2 + 0) * 16 + 4 * g4);
            const f32x4 mr = *reinterpret_cast<const f32x4*>(sc + ((wave * RB + rb) * 2 + 1) * 16 + 4 * g4);
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = mr[e] * ap[rb][e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(cx[e] * ag[rb][e]));
            const int m0 = rb * 16 + 4 * g4;
            bf16* p = m0 < mvalid ? dst + m0 : sink + lane * 4;
            Elem<bf16>::store4(p, 0, o);
        }
        // Stage q + 1 must have landed: after its DMA this wave issued the
        // stores of stage q - 1, the DMA of stage q + 2 and the stores of stage q.
        if (q + 2 < NQ) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(DPW + RB));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(0));
        barrier();
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
    int blocks_per_b;
    if (!incoming) {
        const size_t NN = (size_t)N * N;
        blocks_per_b = (int)((NN + NWV * ROWS - 1) / (NWV * ROWS));
    } else {
        blocks_per_b = ((N + ROWS - 1) / ROWS) * (N / NWV);
    }
    dim3 grid((unsigned)((size_t)B * blocks_per_b));
    hipLaunchKernelGGL((k1_project_fold<D>), grid, dim3(256), 0, s, (const bf16*)z, (const bf16*)mask,
                       (const bf16*)p.w_proj_f, (const bf16*)p.x_proj, p.eps, (bf16*)a, (bf16*)b,
                       (bf16*)p.sink, N, p.C, incoming, blocks_per_b);
    return hipGetLastError();
}

hipError_t launch_project(const Params& p, const void* z, const void* mask, int B, int N,
                          int incoming, void* a_cm, void* b_cm, hipStream_t s)
{
    if (p.dtype == DType::BF16 && p.D == 256)
        return launch_k1_fold<256>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    if (p.dtype == DType::BF16 && p.D == 128)
        return launch_k1_fold<128>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    if (p.dtype == DType::BF16) return launch_k1_d<bf16>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    return launch_k1_d<float>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
}

}  // namespace trimul
