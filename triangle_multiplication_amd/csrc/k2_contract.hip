// k2_contract.hip -- the triangle contraction: for every (batch, channel) slab,
// o[i][j] = sum_k a_cm[i][k] * b_cm[j][k] over k in [0, N), fp32 accumulation
// on matrix cores, one rounding to the storage type at the end.
//
// The projection kernel stores a and b channel-major with k contiguous for both
// directions (the incoming direction's transpose is folded into that store), so
// this is always an "NT" product of two K-contiguous operands.
//
// Tiling: a 256-thread workgroup (4 waves in a 2 x 2 grid) owns a BM x BN tile
// of o; each wave owns (BM/2) x (BN/2) as 16 x 16 MFMA blocks.  K advances 128
// bytes per stage (64 bf16 / 32 fp32), staged through double-buffered LDS with
// the chunk swizzle of trimul_device.hpp; global loads for stage k+1 are in
// flight while stage k is multiplied.  Rows or K chunks past N read as zero, and
// stores past N are skipped, so any N that is a multiple of 8 works.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void k2_contract(const T* __restrict__ A, const T* __restrict__ Bm,
                                                   T* __restrict__ O, int N, int tiles_j)
{
    constexpr int CE = Elem<T>::CE;
    constexpr int KCH = 8;                  // 16-byte chunks per tile row per stage
    constexpr int BK = KCH * CE;            // K elements per stage
    constexpr int WM = BM / 2, WN = BN / 2; // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int A_LD = BM * KCH / 256;    // chunks each thread loads per stage
    constexpr int B_LD = BN * KCH / 256;
    __shared__ u32x4 lds[2][(BM + BN) * KCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t slab = (size_t)N * N;
    const size_t bc = blockIdx.y;
    const T* Ab = A + bc * slab;
    const T* Bb = Bm + bc * slab;
    T* Ob = O + bc * slab;
    const int ti = blockIdx.x / tiles_j, tj = blockIdx.x % tiles_j;
    const int i0 = ti * BM, j0 = tj * BN;

    u32x4 ra[A_LD], rb[B_LD];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gi = i0 + row, gk = k0 + c * CE;
            ra[it] = (gi < N && gk < N) ? ld16(Ab + (size_t)gi * N + gk) : zero;
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gj = j0 + row, gk = k0 + c * CE;
            rb[it] = (gj < N && gk < N) ? ld16(Bb + (size_t)gj * N + gk) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][row * KCH + swz(row, c)] = ra[it];
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][BM * KCH + row * KCH + swz(row, c)] = rb[it];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (N + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kg = 0; kg < KCH / 4; ++kg) {
            const int c = kg * 4 + (lane >> 4);
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                int row = wm * WM + m * 16 + (lane & 15);
                fa[m] = lds[buf][row * KCH + swz(row, c)];
            }
#pragma unroll
            for (int n = 0; n < FN; ++n) {
                int row = wn * WN + n * 16 + (lane & 15);
                fb[n] = lds[buf][BM * KCH + row * KCH + swz(row, c)];
            }
            // Operands swapped (b rows as the MFMA's A): each lane's four results
            // are four consecutive j of one i, so the store is one 4-element run.
#pragma unroll
            for (int m = 0; m < FM; ++m)
#pragma unroll
                for (int n = 0; n < FN; ++n) acc[m][n] = Elem<T>::mma(fb[n], fa[m], acc[m][n]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < FM; ++m) {
        const int i = i0 + wm * WM + m * 16 + (lane & 15);
#pragma unroll
        for (int n = 0; n < FN; ++n) {
            const int j = j0 + wn * WN + n * 16 + 4 * (lane >> 4);
            if (i < N && j < N) Elem<T>::store4(Ob, (size_t)i * N + j, acc[m][n]);
        }
    }
}

template <typename T, int BM, int BN>
static hipError_t launch_k2(const void* a, const void* b, int B, int C, int N, void* o,
                            hipStream_t s)
{
    const int tiles_i = (N + BM - 1) / BM, tiles_j = (N + BN - 1) / BN;
    dim3 grid((unsigned)(tiles_i * tiles_j), (unsigned)(B * C));
    hipLaunchKernelGGL((k2_contract<T, BM, BN>), grid, dim3(256), 0, s,
                       (const T*)a, (const T*)b, (T*)o, N, tiles_j);
    return hipGetLastError();
}

hipError_t launch_contract(const Params& p, const void* a_cm, const void* b_cm, int B, int N,
                           void* o, hipStream_t s)
{
    if (p.dtype == DType::BF16) return launch_k2<bf16, 128, 128>(a_cm, b_cm, B, p.C, N, o, s);
    return launch_k2<float, 128, 128>(a_cm, b_cm, B, p.C, N, o, s);
}

}  // namespace trimul
