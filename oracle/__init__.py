"""fp64 CPU oracle for the SO(2) equivariant message-passing layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product path (the HIP library and its Python binding) never does, and shares
no code, table or constant with it.

Every function follows a passage of the pages it is written from:

* "Distributed Equivariant Graph Neural Networks for Large-Scale Electronic
  Structure Prediction" (pith.science review of arXiv 2507.03840), "What
  carries the argument": the incoming-edge layout, attention and aggregation
  over the edges directed into a node.
* "MALOQ" (arXiv 2606.28911v1): Sec. III (workflow of Fig. 2(a)), Sec. III-B1
  Eq. (1) (Clebsch-Gordan decomposition of Hamiltonian sub-blocks),
  Sec. III-B2 (Matrix <-> Label with orbital templates and padding),
  Sec. III-C1 and Fig. 3(b,c) (Wigner-D rotation of every edge to +y),
  Sec. III-D (messages n_i (+) n_j; target node owns its edges),
  Sec. II-B1 (SO(3) -> SO(2) reduction, eSCN).

Where the pages leave a step open the plainest reading is taken; each such
reading is named in the docstring of the function that takes it.

Parity unpinned: the *choice* of those readings.  The pages print no value
that could decide between equally valid readings of these steps, so the
tests pin each function's arithmetic for the reading taken (invariants,
brute force, closed forms, finite differences), not the reading itself:
  layer.radial_basis (centres and width of the Gaussians),
  layer.gates (radial basis as per-(m, l, channel) input gates),
  layer.trunc_mask (coefficients with |m| > mmax dropped),
  layer.edge_forward (source-then-destination message channels; the
      attention logit from the invariant output channels),
  layer.layer_forward (residual update; the per-edge message as the edge
      irreps of the decode),
  layer.layer_backward (the loss <G, x'>),
  decode.label_layout / labels_from_irreps / label_to_matrix (label order,
      the 2s2p1d basis, no hermiticity symmetrisation),
  so3.real_coupling (the sign rule of the real coupling),
  labels (each element's shells as a subset of one full list, padding at the
      full list's label positions, matrices of a batch back to back, no
      block for edges across structures or with an image shift).

Modules:
  neighbors  -- brute-force periodic / open cutoff graph, destination-sorted CSR
  so3        -- real spherical harmonics, Wigner-D, edge frame, real CG couplings
  layer      -- layer forward and analytic backward
  decode     -- Label -> Matrix: Hamiltonian blocks from irreps
  labels     -- Matrix <-> Label over whole matrices with per-element orbital
                templates (MALOQ Sec. III-B2)
"""
