"""The chunked form of the recurrence on the CPU, fp64, for one head.

TEST INFRASTRUCTURE (see the package docstring). The pages state that the
chunked schedule produces exactly the same state and outputs as the
token-by-token recurrence; these functions write that schedule out so a test
can hold the sequential oracle and the chunk algebra against each other.

Pages (titles), cited by the short name in brackets:
  [family]  "Uma análise das variantes de atenção linear da família DeltaNet",
            section "Chunkwise KDA: reorganizando a recorrência como
            multiplicações de matrizes" and its subsections "Atenuação
            acumulada e erros provisórios", "Restauração das dependências
            causais", "Cálculo do estado ao fim do chunk", "Cálculo de todas
            as saídas dentro do chunk"; section "Pipeline Triton da versão por
            chunks" (decay over a span as a difference of two prefix sums).
  [gdn2]    "Resumo Técnico: Gated DeltaNet-2", section "Treinamento Paralelo
            Eficiente por Blocos" (decay absorbed into the erase factors,
            triangular system (I+T), auxiliary Y on the erase side and U on
            the write side).

[family] writes KDA with the state in R^{d_v x d_k}; here the state is kept
d_k x d_v (S = S'^T) and the erase key e and gated value z of the decoupled
gates replace beta k and beta v, which is the generalisation [gdn2] makes.

Inputs (fp64): q, k, e [T, d_k]; z [T, d_v]; g [T, d_k] the log decay
(scalar decay is passed broadcast to d_k); S0 [d_k, d_v]. Chunk length C >= 1;
the last chunk may be shorter.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _chunks(T, C):
    for c0 in range(0, T, C):
        yield c0, min(T, c0 + C)


def chunked_provisional(q, k, e, z, g, scale, S0, C):
    """[family]'s chunk algorithm: provisional errors, causal coupling rho,
    unit-lower triangular solve, end-of-chunk state, in-chunk outputs."""
    T, dk = k.shape
    dv = z.shape[1]
    S = S0.copy()
    o = np.zeros((T, dv))
    for c0, c1 in _chunks(T, C):
        n = c1 - c0
        # Cumulative log decay from the chunk boundary through token i (inclusive):
        # D_{0:i} = Diag(exp(G_i)); D_{j+1:i} = Diag(exp(G_i - G_j)).
        G = np.cumsum(g[c0:c1], axis=0)
        kc, qc, ec, zc = k[c0:c1], q[c0:c1], e[c0:c1], z[c0:c1]
        # Provisional errors, ignoring the writes earlier in the chunk.
        ubar = np.stack([zc[i] - (np.exp(G[i])[:, None] * S).T @ ec[i] for i in range(n)])
        # rho_ij: how token j's write changes token i's prediction (j < i).
        R = np.zeros((n, n))
        for i in range(n):
            for j in range(i):
                R[i, j] = np.sum(ec[i] * np.exp(G[i] - G[j]) * kc[j])
        # Resolved errors: u_i = ubar_i - sum_{j<i} rho_ij u_j, i.e. (I + R) U = Ubar.
        U = solve_triangular(np.eye(n) + R, ubar, lower=True, unit_diagonal=True)
        # Outputs: chi_ij = scale * q_i^T D_{j+1:i} k_j for j <= i (own write included),
        # plus the read of the entry state decayed to token i.
        for i in range(n):
            acc = scale * (np.exp(G[i])[:, None] * S).T @ qc[i]
            for j in range(i + 1):
                chi = scale * np.sum(qc[i] * np.exp(G[i] - G[j]) * kc[j])
                acc = acc + chi * U[j]
            o[c0 + i] = acc
        # End state: entry state through all the chunk's decays, plus every write
        # carried through the decays after it (keys decayed to the chunk end).
        Kend = kc * np.exp(G[n - 1][None, :] - G)
        S = np.exp(G[n - 1])[:, None] * S + Kend.T @ U
    return o, S


def chunked_wy(q, k, e, z, g, scale, S0, C):
    """[gdn2]'s block algorithm: absorb the cumulative decay into the erase
    factors (E_bar) and solve (I + T) once for the erase side Y and the write
    side U_z; the resolved errors are U = U_z - Y S_c."""
    T, dk = k.shape
    dv = z.shape[1]
    S = S0.copy()
    o = np.zeros((T, dv))
    for c0, c1 in _chunks(T, C):
        n = c1 - c0
        G = np.cumsum(g[c0:c1], axis=0)
        kc, qc, ec, zc = k[c0:c1], q[c0:c1], e[c0:c1], z[c0:c1]
        Ebar = ec * np.exp(G)                 # erase factors with decay absorbed
        Kinv = kc * np.exp(-G)                # keys with the decay divided out
        Tm = np.tril(Ebar @ Kinv.T, k=-1)     # strictly lower coupling
        I = np.eye(n)
        Y = solve_triangular(I + Tm, Ebar, lower=True, unit_diagonal=True)
        Uz = solve_triangular(I + Tm, zc, lower=True, unit_diagonal=True)
        U = Uz - Y @ S
        Qbar = qc * np.exp(G)
        A = np.tril(Qbar @ Kinv.T)            # read coupling, diagonal included
        o[c0:c1] = scale * (Qbar @ S + A @ U)
        Kend = kc * np.exp(G[n - 1][None, :] - G)
        S = np.exp(G[n - 1])[:, None] * S + Kend.T @ U
    return o, S
