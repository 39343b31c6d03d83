// norm_la.hpp -- launch interface of the normalised linear-attention kernels
// (norm_la.hip): the feature-mapped read with a normaliser of the page
// "Linear attention e fast weights", section "Conceito".
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdr {

struct NlaArgs {
    const void *q, *k, *v;   // phi(q), phi(k) [B,T,Hqk,D]; v [B,T,Hv,D] (io dtype)
    const float *S0, *z0;    // [B,Hv,D,D], [B,Hv,D], or null (zeros)
    void *o;                 // [B,T,Hv,D] (io dtype)
    float *ST, *zT;          // [B,Hv,D,D], [B,Hv,D]
    float *ws;               // [B*Hv][P][D*D + D]: per-segment sums, then segment start states
    int B, T, Hqk, Hv, NC, P, L;  // chunks of 64 tokens; P segments of L chunks each
    int z_apart;             // z_T is formed by a pass of its own (z_T == z0 with one segment)
};

// Segments of the sequence run side by side: P of L chunks each (P = 1 for
// short sequences or many heads). At d = 128 the sweep's B * Hv * 2 work
// items of 64 value columns per segment run two per CU, so P is the most
// segments whose sweep fills the 256 CUs in one round (a second, partial
// round would cost a whole segment's walk again); at smaller d, P is such
// that B * Hv * P * (D / 32) workgroups fill the GPU.
inline void nla_segments(int B, int Hv, int D, int NC, int &P, int &L) {
    const long long items = (long long)B * Hv * (D / 32);
    long long p = items <= 0 ? 1 : D == 128 ? 512 / (items / 2) : (2048 + items - 1) / items;
    p = p < 32 ? p : 32;
    p = p < NC / 2 ? p : NC / 2;
    if (p < 2) { P = 1; L = NC; return; }
    L = (int)((NC + p - 1) / p);
    P = (NC + L - 1) / L;
}
inline size_t nla_ws_bytes(int B, int Hv, int D, int NC) {
    int P, L;
    nla_segments(B, Hv, D, NC, P, L);
    return P > 1 ? (size_t)B * Hv * P * ((size_t)D * D + D) * sizeof(float) : 0;
}

// decode: the one-token step (T = 1, ST = S0 and zT = z0 updated in place).
hipError_t launch_nla(int io, int D, const NlaArgs &a, bool decode, hipStream_t s);

}  // namespace gdr
