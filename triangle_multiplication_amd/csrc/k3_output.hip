// k3_output.hip -- LayerNorm_out, output projection and output gate.
//
// For each pair (i, j):  y = LayerNorm_out(o[:, i, j])  (over C),
//   out[i, j, d] = (p_out y)_d * sg((g_out LayerNorm_in(z_ij))_d).
// The gate's LayerNorm_in is recomputed here from z (the same arithmetic the
// projection kernel does) instead of being stored by that kernel: reading z
// once costs less HBM traffic than writing and re-reading a [N, N, D] gate.
//
// Work split: a 256-thread workgroup owns TM consecutive pairs (natural order,
// the same for both directions), each wave ROWS of them.  The o tile [C][TM]
// (channel-major in HBM, runs of TM contiguous pairs) is staged through LDS and
// gathered per lane into MFMA operand layout; LayerNorm statistics come from
// two cross-lane reductions in fp32.  z rows are loaded straight into operand
// registers like in the projection kernel.  Output channels are produced 16 *
// NB at a time from weight rows staged in LDS; the products are computed with
// weights as the MFMA's A operand, so each lane holds four consecutive output
// channels of one pair and stores them as one 4-element run.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

template <typename T, int D, int C>
struct K3Cfg {
    static constexpr int CE = Elem<T>::CE;
    static constexpr int RB = (sizeof(T) == 2) ? 2 : 1;  // 16-row blocks per wave
    static constexpr int ROWS = RB * 16;
    static constexpr int TM = 4 * ROWS;                   // pairs per workgroup
    static constexpr int DCH = D / CE, CCH = C / CE;
    static constexpr int KGD = DCH / 4, KGC = CCH / 4;
    static constexpr int NB = (sizeof(T) == 2 && D % 64 == 0) ? 4 : 2;  // 16-column blocks per weight stage
    static constexpr int NCOL = NB * 16;
    static constexpr int SWD = swz_mask(DCH), SWC = swz_mask(CCH);
    static constexpr int OCH = TM / CE;                   // chunks per o-tile row
};

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void k3_output(
    const T* __restrict__ z, const T* __restrict__ o, const T* __restrict__ Wgo,
    const T* __restrict__ Wpo, const float* __restrict__ lnw_in, const float* __restrict__ lnb_in,
    const float* __restrict__ lnw_out, const float* __restrict__ lnb_out, float eps,
    T* __restrict__ out, int N, int blocks_per_b)
{
    using Cf = K3Cfg<T, D, C>;
    constexpr int CE = Cf::CE, RB = Cf::RB, ROWS = Cf::ROWS, TM = Cf::TM;
    constexpr int DCH = Cf::DCH, CCH = Cf::CCH, KGD = Cf::KGD, KGC = Cf::KGC;
    constexpr int NB = Cf::NB, NCOL = Cf::NCOL, SWD = Cf::SWD, SWC = Cf::SWC, OCH = Cf::OCH;
    __shared__ T otile[C * TM];
    __shared__ u32x4 wgo_s[NCOL * DCH];
    __shared__ u32x4 wpo_s[NCOL * CCH];
    __shared__ float s_wi[D], s_bi[D], s_wo[C], s_bo[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t NN = (size_t)N * N;
    const int bidx = blockIdx.x / blocks_per_b;
    const size_t p0 = (size_t)(blockIdx.x % blocks_per_b) * TM;   // first pair of the tile
    const int tvalid = (int)min((size_t)TM, NN - p0);             // pairs of the tile that exist

    for (int d = tid; d < D; d += 256) { s_wi[d] = lnw_in[d]; s_bi[d] = lnb_in[d]; }
    for (int c = tid; c < C; c += 256) { s_wo[c] = lnw_out[c]; s_bo[c] = lnb_out[c]; }

    // Stage o[:, p0 : p0+TM] into LDS as otile[c][pair].
    const u32x4 zero = {0u, 0u, 0u, 0u};
    {
        const T* ob = o + (size_t)bidx * C * NN + p0;
        u32x4* ot = reinterpret_cast<u32x4*>(otile);
        for (int idx = tid; idx < C * OCH; idx += 256) {
            const int c = idx / OCH, ch = idx % OCH;
            ot[idx] = (ch * CE < tvalid) ? ld16(ob + (size_t)c * NN + ch * CE) : zero;
        }
    }

    // z operand registers for the gate and their LayerNorm_in.
    u32x4 xf[RB][KGD];
    const T* zb = z + ((size_t)bidx * NN) * D;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = wave * ROWS + rb * 16 + (lane & 15);
        const T* zp = zb + (p0 + m) * D;
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg)
            xf[rb][kg] = (m < tvalid) ? ld16(zp + (kg * 4 + (lane >> 4)) * CE) : zero;
    }
    __syncthreads();  // otile and LayerNorm parameters visible

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float v[KGD][CE];
        float s = 0.f;
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg) {
            Elem<T>::unpack(xf[rb][kg], v[kg]);
#pragma unroll
            for (int e = 0; e < CE; ++e) s += v[kg][e];
        }
        const float mu = sum_row_lanes(s) * (1.0f / D);
        float q = 0.f;
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg)
#pragma unroll
            for (int e = 0; e < CE; ++e) { float dl = v[kg][e] - mu; q += dl * dl; }
        const float rstd = rsqrtf(sum_row_lanes(q) * (1.0f / D) + eps);
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg) {
            const int d0 = (kg * 4 + (lane >> 4)) * CE;
            float y[CE];
#pragma unroll
            for (int e = 0; e < CE; ++e) y[e] = (v[kg][e] - mu) * rstd * s_wi[d0 + e] + s_bi[d0 + e];
            xf[rb][kg] = Elem<T>::pack(y);
        }
    }

    // y operand registers: gathered from the o tile, LayerNorm_out over C.
    u32x4 yf[RB][KGC];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = wave * ROWS + rb * 16 + (lane & 15);
        float v[KGC][CE];
        float s = 0.f;
#pragma unroll
        for (int kg = 0; kg < KGC; ++kg) {
            const int c0 = (kg * 4 + (lane >> 4)) * CE;
#pragma unroll
            for (int e = 0; e < CE; ++e) { v[kg][e] = (float)otile[(c0 + e) * TM + m]; s += v[kg][e]; }
        }
        const float mu = sum_row_lanes(s) * (1.0f / C);
        float q = 0.f;
#pragma unroll
        for (int kg = 0; kg < KGC; ++kg)
#pragma unroll
            for (int e = 0; e < CE; ++e) { float dl = v[kg][e] - mu; q += dl * dl; }
        const float rstd = rsqrtf(sum_row_lanes(q) * (1.0f / C) + eps);
#pragma unroll
        for (int kg = 0; kg < KGC; ++kg) {
            const int c0 = (kg * 4 + (lane >> 4)) * CE;
            float y[CE];
#pragma unroll
            for (int e = 0; e < CE; ++e) y[e] = (v[kg][e] - mu) * rstd * s_wo[c0 + e] + s_bo[c0 + e];
            yf[rb][kg] = Elem<T>::pack(y);
        }
    }

    T* ob = out + ((size_t)bidx * NN) * D;
    for (int q = 0; q < D / NCOL; ++q) {
        __syncthreads();  // previous stage fully consumed
        for (int idx = tid; idx < NCOL * DCH; idx += 256) {
            const int row = idx / DCH, c = idx % DCH;
            wgo_s[row * DCH + (c ^ (row & SWD))] = ld16(Wgo + (size_t)(q * NCOL + row) * D + c * CE);
        }
        for (int idx = tid; idx < NCOL * CCH; idx += 256) {
            const int row = idx / CCH, c = idx % CCH;
            wpo_s[row * CCH + (c ^ (row & SWC))] = ld16(Wpo + (size_t)(q * NCOL + row) * C + c * CE);
        }
        __syncthreads();
        f32x4 ag[RB][NB], ay[RB][NB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                ag[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                ay[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg) {
            const int c = kg * 4 + (lane >> 4);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = nb * 16 + (lane & 15);
                const u32x4 fw = wgo_s[row * DCH + (c ^ (row & SWD))];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) ag[rb][nb] = Elem<T>::mma(fw, xf[rb][kg], ag[rb][nb]);
            }
        }
#pragma unroll
        for (int kg = 0; kg < KGC; ++kg) {
            const int c = kg * 4 + (lane >> 4);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = nb * 16 + (lane & 15);
                const u32x4 fw = wpo_s[row * CCH + (c ^ (row & SWC))];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) ay[rb][nb] = Elem<T>::mma(fw, yf[rb][kg], ay[rb][nb]);
            }
        }
        // Lane holds channels q*NCOL + nb*16 + 4*(lane/16) + r of pair rb*16 + lane%16.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int m = wave * ROWS + rb * 16 + (lane & 15);
            if (m < tvalid) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = ay[rb][nb][e] * sigmoidf_(ag[rb][nb][e]);
                    Elem<T>::store4(ob, (p0 + m) * D + q * NCOL + nb * 16 + 4 * (lane >> 4), r);
                }
            }
        }
    }
}

template <typename T, int D, int C>
static hipError_t launch_k3_t(const Params& p, const void* z, const void* o, int B, int N,
                              void* out, hipStream_t s)
{
    using Cf = K3Cfg<T, D, C>;
    const size_t NN = (size_t)N * N;
    const int blocks_per_b = (int)((NN + Cf::TM - 1) / Cf::TM);
    dim3 grid((unsigned)((size_t)B * blocks_per_b));
    hipLaunchKernelGGL((k3_output<T, D, C>), grid, dim3(256), 0, s, (const T*)z, (const T*)o,
                       (const T*)p.w_gout, (const T*)p.w_pout, p.ln_in_w, p.ln_in_b, p.ln_out_w,
                       p.ln_out_b, p.eps, (T*)out, N, blocks_per_b);
    return hipGetLastError();
}

#define TRIMUL_K3_C_CASES(T, D)                                                           \
    switch (p.C) {                                                                        \
    case 32: return launch_k3_t<T, D, 32>(p, z, o, B, N, out, s);                         \
    case 64: return launch_k3_t<T, D, 64>(p, z, o, B, N, out, s);                         \
    case 96: return launch_k3_t<T, D, 96>(p, z, o, B, N, out, s);                         \
    case 128: return launch_k3_t<T, D, 128>(p, z, o, B, N, out, s);                       \
    case 160: return launch_k3_t<T, D, 160>(p, z, o, B, N, out, s);                       \
    case 192: return launch_k3_t<T, D, 192>(p, z, o, B, N, out, s);                       \
    case 224: return launch_k3_t<T, D, 224>(p, z, o, B, N, out, s);                       \
    case 256: return launch_k3_t<T, D, 256>(p, z, o, B, N, out, s);                       \
    default: return hipErrorInvalidValue;                                                 \
    }

template <typename T>
static hipError_t launch_k3_d(const Params& p, const void* z, const void* o, int B, int N,
                              void* out, hipStream_t s)
{
    switch (p.D) {
    case 32: TRIMUL_K3_C_CASES(T, 32)
    case 64: TRIMUL_K3_C_CASES(T, 64)
    case 96: TRIMUL_K3_C_CASES(T, 96)
    case 128: TRIMUL_K3_C_CASES(T, 128)
    case 160: TRIMUL_K3_C_CASES(T, 160)
    case 192: TRIMUL_K3_C_CASES(T, 192)
    case 224: TRIMUL_K3_C_CASES(T, 224)
    case 256: TRIMUL_K3_C_CASES(T, 256)
    default: return hipErrorInvalidValue;
    }
}

bool output_supported(int D, int C, DType)
{
    return D >= 32 && D <= 256 && D % 32 == 0 && C >= 32 && C <= 256 && C % 32 == 0;
}

hipError_t launch_output(const Params& p, const void* z, const void* o, int B, int N, void* out,
                         hipStream_t s)
{
    if (p.dtype == DType::BF16) return launch_k3_d<bf16>(p, z, o, B, N, out, s);
    return launch_k3_d<float>(p, z, o, B, N, out, s);
}

}  // namespace trimul
