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

// Slab bc of o under an OutputSrc: the first `split` slabs are contiguous at
// o_lo; the rest sit at o_hi with their own stride (the workspace-lean layout
// puts them over operand slabs the contraction has finished with).
template <typename T>
__device__ inline const T* o_slab(const OutputSrc& os, size_t bc, size_t NN)
{
    return bc < (size_t)os.split ? (const T*)os.o_lo + bc * NN
                                 : (const T*)os.o_hi + (bc - (size_t)os.split) * os.hi_stride;
}

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void k3_output(
    const T* __restrict__ z, const OutputSrc osrc, const T* __restrict__ Wgo,
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
        u32x4* ot = reinterpret_cast<u32x4*>(otile);
        for (int idx = tid; idx < C * OCH; idx += 256) {
            const int c = idx / OCH, ch = idx % OCH;
            const T* oc = o_slab<T>(osrc, (size_t)bidx * C + c, NN);
            ot[idx] = (ch * CE < tvalid) ? ld16(oc + p0 + ch * CE) : zero;
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

// ---------------------------------------------------------------------------
// bf16 path for D = C in {128, 256}: persistent, LayerNorm folded into the
// output GEMMs, weights resident in registers, activations in an LDS ring.
//
// Both LayerNorms are applied algebraically instead of element by element.
// For a row v of length L with mean mu and rstd = 1 / sqrt(var + eps), and a
// weight row W acting on gamma * (v - mu) * rstd + beta:
//   W (gamma (v - mu) rstd + beta) = rstd (W' v - mu S + T sd),
//   W' = gamma-scaled W (rounded to bf16), S = sum of W' row, T = W beta,
//   sd = 1 / rstd.
// The matrix cores multiply W' with the raw bf16 rows of z and o, and one
// extra MFMA per output block adds -mu S + T sd from a K-group whose lane
// group 0 holds mu and sd split into bf16 high and low parts (six products:
// mu_h S_h, mu_h S_l, mu_l S_h, sd_h T_h, sd_h T_l, sd_l T_h; the host
// supplies S and T split the same way) and whose other lanes hold zeros.  It
// is the first MFMA of each accumulation chain.  (The 16x16x16 bf16 MFMA
// would need fewer registers, but this compiler under-counts its latency on
// gfx950 and lets a VALU read its result too early.)  Statistics take one pass with
// v_dot2_f32_bf16 (sum and sum of squares, var = E[v^2] - mu^2 in fp32).
// The epilogue is then out = (rstd_o acc_p) / (1 + 2^(-log2(e) rstd_x acc_g)).
//
// Persistent workgroups (one of 8 waves per CU at D = 256, two of 4 waves at
// D = 128) walk 32-pair tiles of a contiguous range of pairs; the two halves
// of each 64-pair run go to the same workgroup back to back, so the second
// half of every 128-byte line of o is an L2 hit.  Each wave owns two 16-row blocks of the D output channels
// (rows interleaved so that a lane's results are eight consecutive channels)
// and holds those rows of W'_g and W'_p in registers for the whole kernel.  A ring of four LDS slots, filled by
// global->LDS DMA three tiles ahead, holds per tile
//   z: 32 rows of 2D bytes, 16-byte chunk c of row p stored at c ^ (p % 16);
//   o: C channel rows of 64 bytes (32 pairs), 32-byte half h of row c stored at
//      h ^ ((c >> 3) & 1), so ds_read_b64_tr_b16 reads of a 32-lane half touch
//      distinct banks.
// Per tile t: waves 0..3 compute the statistics of tile t + 1 (one of the two
// 16-pair blocks of z or of o each) into a double-buffered LDS record; then all
// waves run the MFMAs and the epilogue of tile t; one barrier ends the tile.
// ---------------------------------------------------------------------------
namespace k3f {
constexpr int TM = 32, NB = TM / 16, NS = 4;
// Waves per workgroup: 8 at D = 256 (one workgroup per CU), 4 at D = 128
// (two per CU), so that every wave owns two paired 16-row blocks.
constexpr int waves_for(int D) { return D >= 256 ? 8 : 4; }
constexpr float LOG2E = 1.4426950408889634f;

template <int D, int C>
struct Cfg {
    static constexpr int KGD = D / 32, KGC = C / 32;
    static constexpr int NW = waves_for(D);
    static constexpr int RBT = D / 16, RBW = RBT / NW;      // 16-row output blocks (per wave)
    static constexpr int ZB = TM * D * 2, OB = C * TM * 2;   // slot bytes of z and of o
    static constexpr int SLOT = ZB + OB;
    static constexpr int ZDMA = ZB / 1024, DMA_ALL = (ZB + OB) / 1024;
    static constexpr int DPW = DMA_ALL / NW;                  // 1 KB DMA instructions per wave per tile
    // With two row blocks per wave they are interleaved so that each lane's
    // eight results are eight consecutive channels (one 16-byte store).
    static constexpr bool PAIRED = RBW == 2;
    static constexpr int STORES = PAIRED ? NB : NB * RBW;     // global stores per wave per tile
    static constexpr int FRAG = 1024;                         // one extra K-group fragment
    static constexpr int STAT = 4 * FRAG + 4 * 64;            // [kind][block] fragments + scales
    static constexpr int LDS = NS * SLOT + 2 * STAT;
    static_assert(D % 32 == 0 && C % 32 == 0 && D >= 128 && RBT % NW == 0, "widths");
    static_assert(DMA_ALL % NW == 0 && ZB % 1024 == 0 && OB % 1024 == 0, "DMA split");
    static_assert(LDS <= 160 * 1024, "LDS");
};
}  // namespace k3f

// The o operand of one 16-pair block, KG fragments of 16 bytes, each made of two
// transposing 8-byte LDS reads at base + 2048 kg and base + 2048 kg + 256.  One
// asm block issues all of them and waits for them: the compiler places a wait
// for every outstanding global->LDS DMA before each transposing-read builtin
// (it cannot tell that the read does not touch the slots in flight), which
// would drain the prefetch ring on every tile.  The slots read here have
// landed by the kernel's own vmcnt waits and barriers.
template <int KG> struct OFrags;
#define TRIMUL_TR2(i, off) "ds_read_b64_tr_b16 %" #i ", %[a] offset:" #off "\n\t"
template <> struct OFrags<8> {
    __device__ static inline void read(uint32_t a, u32x4 (&y)[8]) {
        u32x2 r[16];
        asm volatile(TRIMUL_TR2(0, 0) TRIMUL_TR2(1, 256) TRIMUL_TR2(2, 2048) TRIMUL_TR2(3, 2304)
                     TRIMUL_TR2(4, 4096) TRIMUL_TR2(5, 4352) TRIMUL_TR2(6, 6144) TRIMUL_TR2(7, 6400)
                     TRIMUL_TR2(8, 8192) TRIMUL_TR2(9, 8448) TRIMUL_TR2(10, 10240) TRIMUL_TR2(11, 10496)
                     TRIMUL_TR2(12, 12288) TRIMUL_TR2(13, 12544) TRIMUL_TR2(14, 14336) TRIMUL_TR2(15, 14592)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                       "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
                       "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
                     : [a] "v"(a));
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = u32x4{r[2 * k][0], r[2 * k][1], r[2 * k + 1][0], r[2 * k + 1][1]};
    }
};
template <> struct OFrags<4> {
    __device__ static inline void read(uint32_t a, u32x4 (&y)[4]) {
        u32x2 r[8];
        asm volatile(TRIMUL_TR2(0, 0) TRIMUL_TR2(1, 256) TRIMUL_TR2(2, 2048) TRIMUL_TR2(3, 2304)
                     TRIMUL_TR2(4, 4096) TRIMUL_TR2(5, 4352) TRIMUL_TR2(6, 6144) TRIMUL_TR2(7, 6400)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                       "=&v"(r[6]), "=&v"(r[7])
                     : [a] "v"(a));
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = u32x4{r[2 * k][0], r[2 * k][1], r[2 * k + 1][0], r[2 * k + 1][1]};
    }
};
template <> struct OFrags<6> {
    __device__ static inline void read(uint32_t a, u32x4 (&y)[6]) {
        u32x2 r[12];
        asm volatile(TRIMUL_TR2(0, 0) TRIMUL_TR2(1, 256) TRIMUL_TR2(2, 2048) TRIMUL_TR2(3, 2304)
                     TRIMUL_TR2(4, 4096) TRIMUL_TR2(5, 4352) TRIMUL_TR2(6, 6144) TRIMUL_TR2(7, 6400)
                     TRIMUL_TR2(8, 8192) TRIMUL_TR2(9, 8448) TRIMUL_TR2(10, 10240) TRIMUL_TR2(11, 10496)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                       "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
                     : [a] "v"(a));
#pragma unroll
        for (int k = 0; k < 6; ++k) y[k] = u32x4{r[2 * k][0], r[2 * k][1], r[2 * k + 1][0], r[2 * k + 1][1]};
    }
};
template <> struct OFrags<2> {
    __device__ static inline void read(uint32_t a, u32x4 (&y)[2]) {
        u32x2 r[4];
        asm volatile(TRIMUL_TR2(0, 0) TRIMUL_TR2(1, 256) TRIMUL_TR2(2, 2048) TRIMUL_TR2(3, 2304)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                     : [a] "v"(a));
#pragma unroll
        for (int k = 0; k < 2; ++k) y[k] = u32x4{r[2 * k][0], r[2 * k][1], r[2 * k + 1][0], r[2 * k + 1][1]};
    }
};
#undef TRIMUL_TR2

template <int D, int C>
__global__ __launch_bounds__(k3f::waves_for(D) * 64) void k3_output_fold(
    const bf16* __restrict__ z, const OutputSrc osrc, const bf16* __restrict__ Wg,
    const bf16* __restrict__ Wp, const bf16* __restrict__ Xg, const bf16* __restrict__ Xp,
    float eps, bf16* __restrict__ out, int N, int n_super)
{
    using namespace k3f;
    using Cf = Cfg<D, C>;
    constexpr int KGD = Cf::KGD, KGC = Cf::KGC, RBW = Cf::RBW;
    constexpr int ZB = Cf::ZB, SLOT = Cf::SLOT, FRAG = Cf::FRAG, STAT = Cf::STAT, NW = Cf::NW;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cf::LDS];
    unsigned char* ring = smem;
    unsigned char* stat = smem + NS * SLOT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const size_t NN = (size_t)N * N;
    const int G = gridDim.x, g = blockIdx.x;
    // This workgroup's tiles: 64-pair runs, each as two 32-pair halves back to
    // back (the second half of each 128-byte line of o is then an L2 hit).
    // At D = 256 the workgroups walk runs g, g + G, ..., all on one moving
    // window (1.5-3 % faster there than the contiguous ranges below).  At D =
    // 128 each workgroup walks one contiguous range of runs, so it streams its
    // own stretch of z, out and each channel of o (6-9 % faster than the
    // moving window with two workgroups per CU, the same with one); the walk
    // starts at a position rotated by 97 g runs within the range and wraps:
    // with aligned starts, the lines the workgroups of an XCD read at the same
    // time sat at power-of-two distances and evicted each other from L2, so a
    // third of o's lines were fetched twice.  G <= n_super, so every
    // workgroup has at least one run.
    constexpr bool WINDOW = D >= 256;
    const long long s_begin = WINDOW ? g : (long long)g * n_super / G;
    const int n_runs = WINDOW ? (int)((n_super - g + G - 1) / G)
                              : (int)((long long)(g + 1) * n_super / G - s_begin);
    const int n_tiles = 2 * n_runs;
    const int rot = (WINDOW || n_runs == 0) ? 0 : (int)(((long long)g * 97) % n_runs);
    auto tile_p0 = [&](int it) -> size_t {
        long long run;
        if constexpr (WINDOW) {
            run = s_begin + (long long)(it >> 1) * G;
        } else {
            int r = (it >> 1) + rot;
            if (r >= n_runs) r -= n_runs;
            run = s_begin + r;
        }
        return it < n_tiles ? ((size_t)run * 64 + (it & 1) * 32) : 0;
    };

    // Weight rows of this wave (MFMA A operand: lane = row l16 of the block,
    // chunk g4 of each K-group); the extra K-group uses lanes g4 == 0.
    u32x4 wg[RBW][KGD], wp[RBW][KGC];
    u32x4 xg[RBW], xp[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        // Output channel of MFMA row l16 of block r: with paired blocks, rows
        // 4k + e of block r give channel 32 wave + 8k + 4r + e.
        const int d = Cf::PAIRED ? 32 * wave + 8 * (l16 >> 2) + 4 * r + (l16 & 3) : (wave + r * NW) * 16 + l16;
#pragma unroll
        for (int kg = 0; kg < KGD; ++kg) wg[r][kg] = ld16(Wg + (size_t)d * D + (kg * 4 + g4) * 8);
#pragma unroll
        for (int kg = 0; kg < KGC; ++kg) wp[r][kg] = ld16(Wp + (size_t)d * C + (kg * 4 + g4) * 8);
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
        xg[r] = g4 == 0 ? ld16(Xg + d * 8) : zero4;
        xp[r] = g4 == 0 ? ld16(Xp + d * 8) : zero4;
    }

    // DMA of tile it into ring slot it % NS.  Instruction q covers 1 KB of the
    // slot; lane l fills its 16 bytes.  Phantom tiles (past the end) re-read
    // tile 0 so that every wave issues the same count.  z is read with the
    // non-temporal hint (each row is read once); o is not, since the second
    // half of each of its 128-byte lines is read by the next tile from L2.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_ring = lds_addr_of(ring);
    auto issue = [&](int it) {
        const size_t p0 = tile_p0(it);
        const size_t bidx = p0 / NN, pin = p0 % NN;
        const uint32_t sl = lds_ring + (uint32_t)((it & (NS - 1)) * SLOT);
        int ln = threadIdx.x & 63;      // opaque: keeps per-lane offsets out of loop-carried registers
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < Cf::DPW; ++i) {
            const int q = wave_s + i * NW;
            if (q < Cf::ZDMA) {
                const int byte = q * 1024 + ln * 16;
                const int row = byte / (D * 2), pch = (byte % (D * 2)) / 16;
                const bf16* src = z + (p0 + row) * D + (pch ^ (row & 15)) * 8;
                dma16_to_lds_nt(src, sl + (uint32_t)(q * 1024));
            } else {
                const int qo = q - Cf::ZDMA;
                const int c = qo * 16 + (ln >> 2), pc = ln & 3;
                const int half = (pc >> 1) ^ ((c >> 3) & 1);
                const bf16* src = o_slab<bf16>(osrc, bidx * C + c, NN) + pin + half * 16 + (pc & 1) * 8;
                dma16_to_lds(src, sl + (uint32_t)(ZB + qo * 1024));
            }
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Fragment addressing.  z, block bb, K-group kg: lane reads chunk
    // (4 kg + g4) ^ l16 of row 16 bb + l16, i.e. zb[kg & 3] + 256 (kg >> 2) + 32 D bb.
    int zb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zb[j] = l16 * (2 * D) + ((g4 ^ (l16 & 3)) * 16) + ((j ^ (l16 >> 2)) << 6);
    // o, block bb, K-group kg, half hh: channel row kg*32 + 8 g4 + 4 hh + l16/4,
    // pairs 16 bb + 4 (l16 % 4) .. +3, i.e. ob_[bb] + 256 hh + 2048 kg.
    int obb[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
        obb[bb] = (g4 * 8 + (l16 >> 2)) * 64 + ((bb ^ (g4 & 1)) * 32) + (l16 & 3) * 8;
    auto zfrag = [&](const unsigned char* sl, int bb, int kg) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(sl + zb[kg & 3] + 256 * (kg >> 2) + 32 * D * bb);
    };
    // All KGC o fragments of block bb (OFrags: one asm block, waited for).
    auto ofrags = [&](const unsigned char* sl, int bb, u32x4 (&yf)[KGC]) {
        const uint32_t a = lds_addr_of(sl + ZB + obb[bb]);
        OFrags<KGC>::read(a, yf);
    };

    // Statistics of one 16-pair block of tile it (waves 0..3: kind = wave / 2
    // selects z or o, bb = wave % 2), written to record it % 2.
    auto stats = [&](int it) {
        const unsigned char* sl = ring + (it & (NS - 1)) * SLOT;
        unsigned char* st = stat + (it & 1) * STAT;
        const int kind = wave >> 1, bb = wave & 1;
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
        float s1 = 0.f, s2 = 0.f;
        auto acc = [&](u32x4 v) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                // Copy the element out first: bit_cast of a vector-element
                // lvalue reads element 0 with this compiler.
                const uint32_t w = v[h];
                const bf16x2 x = __builtin_bit_cast(bf16x2, w);
                s1 = __builtin_amdgcn_fdot2_f32_bf16(x, one2, s1, false);
                s2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, s2, false);
            }
        };
        if (kind == 0) {
#pragma unroll
            for (int kg = 0; kg < KGD; ++kg) acc(zfrag(sl, bb, kg));
        } else {
            u32x4 yf[KGC];
            ofrags(sl, bb, yf);
#pragma unroll
            for (int kg = 0; kg < KGC; ++kg) acc(yf[kg]);
        }
        s1 = sum_row_lanes(s1);
        s2 = sum_row_lanes(s2);
        const float invL = kind == 0 ? 1.0f / D : 1.0f / C;
        const float mu = s1 * invL;
        const float ve = fmaxf(s2 * invL - mu * mu, 0.f) + eps;
        const float rstd = rsqrtf(ve);
        const float sd = ve * rstd;
        const __bf16 nmh = (__bf16)(-mu), nml = (__bf16)(-mu - (float)nmh);
        const __bf16 sdh = (__bf16)sd, sdl = (__bf16)(sd - (float)sdh);
        const __bf16 zr = (__bf16)0.0f;
        bf16x8 f = {zr, zr, zr, zr, zr, zr, zr, zr};
        if (g4 == 0) f = bf16x8{nmh, nmh, nml, sdh, sdh, sdl, zr, zr};
        *reinterpret_cast<bf16x8*>(st + (kind * NB + bb) * FRAG + lane * 16) = f;
        if (g4 == 0)
            *reinterpret_cast<float*>(st + 4 * FRAG + (kind * NB + bb) * 64 + l16 * 4) =
                kind == 0 ? -rstd * LOG2E : rstd;
    };

    // MFMAs and epilogue of tile it.
    auto compute = [&](int it) {
        const unsigned char* sl = ring + (it & (NS - 1)) * SLOT;
        const unsigned char* st = stat + (it & 1) * STAT;
        bf16* ob = out + tile_p0(it) * D;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            f32x4 ag[RBW], ay[RBW];
            u32x4 yfs[KGC];
            ofrags(sl, bb, yfs);
            const u32x4 xe = *reinterpret_cast<const u32x4*>(st + bb * FRAG + lane * 16);
            const u32x4 ye = *reinterpret_cast<const u32x4*>(st + (NB + bb) * FRAG + lane * 16);
#pragma unroll
            for (int r = 0; r < RBW; ++r) {
                const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
                ag[r] = Elem<bf16>::mma(xg[r], xe, z4);
                ay[r] = Elem<bf16>::mma(xp[r], ye, z4);
            }
#pragma unroll
            for (int kg = 0; kg < KGD; ++kg) {
                const u32x4 xf = zfrag(sl, bb, kg);
#pragma unroll
                for (int r = 0; r < RBW; ++r) ag[r] = Elem<bf16>::mma(wg[r][kg], xf, ag[r]);
            }
#pragma unroll
            for (int kg = 0; kg < KGC; ++kg) {
                const u32x4 yf = yfs[kg];
#pragma unroll
                for (int r = 0; r < RBW; ++r) ay[r] = Elem<bf16>::mma(wp[r][kg], yf, ay[r]);
            }
            const float cx = *reinterpret_cast<const float*>(st + 4 * FRAG + bb * 64 + l16 * 4);
            const float ro = *reinterpret_cast<const float*>(st + 4 * FRAG + (NB + bb) * 64 + l16 * 4);
            // Lane holds, for pair 16*bb + l16, output channels 32 wave + 8 g4 +
            // 4r + e (paired blocks) or (wave + 8r)*16 + 4 g4 + e.
            if constexpr (Cf::PAIRED) {
                bf16x8 h;
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        h[4 * r + e] = (bf16)(ro * ay[r][e] *
                                              __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(cx * ag[r][e])));
                *reinterpret_cast<bf16x8*>(ob + (size_t)(bb * 16 + l16) * D + 32 * wave + 8 * g4) = h;
            } else {
#pragma unroll
                for (int r = 0; r < RBW; ++r) {
                    f32x4 res;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        res[e] = ro * ay[r][e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(cx * ag[r][e]));
                    Elem<bf16>::store4(ob, (size_t)(bb * 16 + l16) * D + (wave + r * NW) * 16 + 4 * g4, res);
                }
            }
        }
    };

    issue(0);
    issue(1);
    issue(2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(2 * Cf::DPW));   // tile 0 landed (own share)
    barrier();                                                   // ... everyone's
    if (wave < 4) stats(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(Cf::DPW));       // tile 1 landed
    barrier();
    for (int it = 0; it < n_tiles; ++it) {
        issue(it + 3);                 // into the slot tile it - 1 used
        if (wave < 4) stats(it + 1);
        compute(it);
        // Tile it + 2 must have landed: after its DMA this wave issued at most
        // the stores of tiles it - 1 and it and the DMA of tile it + 3; waiting
        // also for the stores of tile it - 1 costs nothing.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0(Cf::DPW + Cf::STORES));
        barrier();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no DMA may outlive the workgroup
}

template <typename T, int D, int C>
static hipError_t launch_k3_t(const Params& p, const void* z, const OutputSrc& o, int B, int N,
                              void* out, hipStream_t s)
{
    using Cf = K3Cfg<T, D, C>;
    const size_t NN = (size_t)N * N;
    const int blocks_per_b = (int)((NN + Cf::TM - 1) / Cf::TM);
    dim3 grid((unsigned)((size_t)B * blocks_per_b));
    hipLaunchKernelGGL((k3_output<T, D, C>), grid, dim3(256), 0, s, (const T*)z, o,
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

template <int D, int C>
static hipError_t launch_k3_fold(const Params& p, const void* z, const OutputSrc& o, int B, int N,
                                 void* out, hipStream_t s)
{
    const long long n_super = (long long)B * N * N / 64;   // N % 8 == 0, so N*N % 64 == 0
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    constexpr int NW = k3f::Cfg<D, C>::NW;
    // Workgroups resident per CU: 8 waves' worth, as far as the LDS ring allows.
    constexpr int per_cu = (8 / NW) < (160 * 1024) / k3f::Cfg<D, C>::LDS ? (8 / NW) : (160 * 1024) / k3f::Cfg<D, C>::LDS;
    static_assert(per_cu >= 1, "LDS");
    const long long slots = (long long)cus * per_cu;          // workgroups resident at once
    const long long grid = n_super < slots ? n_super : slots;
    hipLaunchKernelGGL((k3_output_fold<D, C>), dim3((unsigned)grid), dim3(NW * 64), 0, s, (const bf16*)z,
                       o, (const bf16*)p.w_gout_f, (const bf16*)p.w_pout_f,
                       (const bf16*)p.x_gout, (const bf16*)p.x_pout, p.eps, (bf16*)out, N,
                       (int)n_super);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_k3_d(const Params& p, const void* z, const OutputSrc& o, int B, int N,
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

hipError_t launch_output(const Params& p, const void* z, const OutputSrc& o, int B, int N, void* out,
                         hipStream_t s)
{
    if (p.dtype == DType::BF16 && p.D == 256 && p.C == 256)
        return launch_k3_fold<256, 256>(p, z, o, B, N, out, s);
    if (p.dtype == DType::BF16 && p.D == 256 && p.C == 128)
        return launch_k3_fold<256, 128>(p, z, o, B, N, out, s);
    if (p.dtype == DType::BF16 && p.D == 128) {
        switch (p.C) {
        case 64: return launch_k3_fold<128, 64>(p, z, o, B, N, out, s);
        case 128: return launch_k3_fold<128, 128>(p, z, o, B, N, out, s);
        case 192: return launch_k3_fold<128, 192>(p, z, o, B, N, out, s);
        case 256: return launch_k3_fold<128, 256>(p, z, o, B, N, out, s);
        default: break;
        }
    }
    if (p.dtype == DType::BF16) return launch_k3_d<bf16>(p, z, o, B, N, out, s);
    return launch_k3_d<float>(p, z, o, B, N, out, s);
}

}  // namespace trimul
