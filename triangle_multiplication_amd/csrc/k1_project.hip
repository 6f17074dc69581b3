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

hipError_t launch_project(const Params& p, const void* z, const void* mask, int B, int N,
                          int incoming, void* a_cm, void* b_cm, hipStream_t s)
{
    if (p.dtype == DType::BF16) return launch_k1_d<bf16>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
    return launch_k1_d<float>(p, z, mask, B, N, incoming, a_cm, b_cm, s);
}

}  // namespace trimul
