"""One DDTree verify round on the GPU: tree build -> every layer of the hybrid
stack -> greedy tree walk -> accepted-path commit, all enqueued on the current
stream through libddt (no host synchronisation inside a round).

Sources: "DDTree on vLLM: candid research notes", section "Why hybrid attention
makes it hard" (tree attention, branch-local recurrent state, accepted-path
commit); "The architecture of speculation", section "The DDTree Integration
Challenge" (drafting, tree construction, tree attention, compaction); "From DDTree
to drafter training", section "The Architecture of DDTree".

There are no dense projections between layers: every layer consumes its own
inputs (queries / tree keys and values for attention, x, v, beta, g for GDN), so
a round exercises exactly the kernels of the verify path.  The round's bonus token
is fed back as the next round's root token, and each commit grows the prefix.
"""

from dataclasses import dataclass, field

import torch

from . import ddt


@dataclass
class HybridConfig:
    n: int = 8                 # sequences
    V: int = 151936            # vocabulary
    L: int = 15                # drafter depth
    B: int = 64                # tree budget (non-root nodes)
    K: int = 0                 # candidates per depth (0 = B)
    prefix: int = 16384        # committed prefix at the first round
    extra_cap: int = 1024      # cache rows beyond the prefix (room for commits)
    n_attn: int = 16
    n_gdn: int = 48
    Hq: int = 24
    Hkv: int = 4
    D: int = 256
    H: int = 32
    dk: int = 128
    W: int = 4
    dtype: torch.dtype = torch.bfloat16
    pattern: list = field(default_factory=list)  # "gdn"/"attn" per layer; default [gdn, gdn, gdn, attn]*
    replay: bool = False       # store no per-node GDN state; the commit replays the accepted path
    rope: tuple = None         # (rot_dim, theta): attention inputs are pre-rotation, RoPE at prefix + depth
    page_size: int = 0         # > 0: the committed KV lives in pages of this many positions (block table)
    sampled: bool = False      # the walk over sampled target tokens (gumbel noise + per-sequence temperature)
    # stored states, bf16: each GDN layer's node-state write (ddt_gdn_tree_states) runs on a
    # second stream beside the next GDN layers, joined before each attention layer and the
    # commit (one workspace per GDN layer). Off by default: the state writes fill every CU,
    # so the next chunk kernel waits for them anyway and the round gains nothing.
    overlap_states: bool = False

    def layer_pattern(self):
        if self.pattern:
            return list(self.pattern)
        out, a, g = [], 0, 0
        while a < self.n_attn or g < self.n_gdn:
            for _ in range(3):
                if g < self.n_gdn:
                    out.append("gdn")
                    g += 1
            if a < self.n_attn:
                out.append("attn")
                a += 1
        return out

    @property
    def T(self):
        return self.B + 1

    @property
    def C(self):
        return 2 * self.H * self.dk

    @property
    def Pmax(self):
        return self.prefix + self.extra_cap


class HybridVerifyStep:
    """Device buffers of a hybrid verify round and the round itself.

    Inputs are filled by the caller (``fill_*`` helpers below use the device RNG);
    outputs and workspaces are allocated once here.
    """

    def __init__(self, cfg: HybridConfig, device="cuda:0"):
        self.cfg = c = cfg
        self.dev = dev = torch.device(device)
        n, T, dt = c.n, c.T, c.dtype
        e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)
        self.draft_logits = e(n, c.L, c.V)
        self.target_logits = e(n, T, c.V)
        self.root_token = torch.zeros(n, dtype=torch.int32, device=dev)
        self.prefix_len = torch.full((n,), c.prefix, dtype=torch.int32, device=dev)
        self.block_table = None
        if c.page_size:
            # pages of every sequence scattered over a shared pool (a seeded permutation,
            # with spare pages), as a serving engine's allocator would leave them
            assert c.Pmax % c.page_size == 0, "capacity must be whole pages"
            maxb = c.Pmax // c.page_size
            self.num_pages = n * maxb + 8
            g = torch.Generator()
            g.manual_seed(1234)
            perm = torch.randperm(self.num_pages, generator=g)[: n * maxb]
            self.block_table = perm.view(n, maxb).to(torch.int32).to(dev)
            cache = lambda: e(self.num_pages, c.Hkv, c.page_size, c.D)
        else:
            cache = lambda: e(n, c.Hkv, c.Pmax, c.D)
        self.attn = [dict(q=e(n, T, c.Hq, c.D), k_tree=e(n, c.Hkv, T, c.D), v_tree=e(n, c.Hkv, T, c.D),
                          k_cache=cache(), v_cache=cache(), out=e(n, T, c.Hq, c.D)) for _ in range(c.n_attn)]
        if c.rope:
            # the tree rows' keys and values as a projection writes them (token-major, before
            # rotation); k_tree / v_tree become outputs of the attention call
            for a in self.attn:
                a["k_new"] = e(n, T, c.Hkv, c.D)
                a["v_new"] = e(n, T, c.Hkv, c.D)
        self.gdn = [dict(x=e(n, T, c.C), v=e(n, T, c.H, c.dk), beta=e(n, T, c.H, dtype=torch.float32),
                         g=e(n, T, c.H, dtype=torch.float32), S=e(n, c.H, c.dk, c.dk, dtype=torch.float32),
                         conv_state=e(n, c.W - 1, c.C), conv_w=e(c.C, c.W, dtype=torch.float32),
                         out=({"o": e(n, T, c.H, c.dk), "S_scratch": None, "conv_scratch": None} if c.replay else
                              {"o": e(n, T, c.H, c.dk), "S_scratch": e(n, T, c.H, c.dk, c.dk, dtype=torch.float32),
                               "conv_scratch": e(n, T, c.W - 1, c.C)}))
                    for _ in range(c.n_gdn)]
        self.tree = {"tok": e(n, T, dtype=torch.int32), "parent": e(n, T, dtype=torch.int32),
                     "depth": e(n, T, dtype=torch.int32), "score": e(n, T, dtype=torch.float32),
                     "anc": e(n, T, dtype=torch.int64)}
        self.acc = {"acc_rows": e(n, c.L + 1, dtype=torch.int32), "acc_len": e(n, dtype=torch.int32),
                    "bonus": e(n, dtype=torch.int32)}
        if c.sampled:
            # the draws' noise for a round (the caller refreshes it between rounds) and temperatures
            self.gumbel = e(n, T, c.V, dtype=torch.float32)
            self.temperature = torch.ones(n, dtype=torch.float32, device=dev)
        u8 = lambda nb: torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        self.ws_build = u8(ddt.build_tree_workspace(n, c.L, c.V, c.B, c.K))
        assert not (c.rope and c.page_size), "RoPE inside the call is built for the contiguous cache"
        self.ws_attn = u8((ddt.tree_attn_rope_workspace if c.rope else ddt.tree_attn_workspace)(
            n, c.B, c.Hq, c.Hkv, c.D, c.Pmax, dt))
        self.ws_acc = u8(ddt.tree_accept_workspace(n, c.B, c.V))
        self.ws_gdn = u8(ddt.gdn_tree_step_workspace(n, c.B, c.H, c.dk))
        self.ws_gdn_layers = None  # per-layer workspaces of the overlapped state writes
        self.side = None
        self.pattern = c.layer_pattern()

    def set_mode(self, replay=None, rope=False):
        """Switch the GDN commit mode (replay) and/or the attention input mode (rope:
        None for post-rotation inputs, (rot_dim, theta) for RoPE inside the call).  Buffers
        a mode needs are allocated here; a newly needed k_new / v_new takes the current
        tree keys / values (token-major), so the data stays that of the workload."""
        c = self.cfg
        if replay is not None:
            c.replay = bool(replay)
            if not c.replay:
                for g in self.gdn:
                    if g["out"]["S_scratch"] is None:
                        g["out"]["S_scratch"] = torch.empty(c.n, c.T, c.H, c.dk, c.dk, dtype=torch.float32,
                                                            device=self.dev)
                        g["out"]["conv_scratch"] = torch.empty(c.n, c.T, c.W - 1, c.C, dtype=c.dtype, device=self.dev)
        if rope is not False:
            assert not (rope and c.page_size), "RoPE inside the call is built for the contiguous cache"
            c.rope = rope
            if rope:
                for a in self.attn:
                    if "k_new" not in a:
                        a["k_new"] = a["k_tree"].transpose(1, 2).contiguous()
                        a["v_new"] = a["v_tree"].transpose(1, 2).contiguous()
            nb = (ddt.tree_attn_rope_workspace if c.rope else ddt.tree_attn_workspace)(
                c.n, c.B, c.Hq, c.Hkv, c.D, c.Pmax, c.dtype)
            if self.ws_attn.numel() < nb:
                self.ws_attn = torch.empty(nb, dtype=torch.uint8, device=self.dev)

    # ------------------------------------------------------------ the round
    def build(self):
        c = self.cfg
        ddt.build_tree(self.draft_logits, c.B, self.root_token, K=c.K, ws=self.ws_build, out=self.tree)

    def overlapping(self):
        c = self.cfg
        return c.overlap_states and not c.replay and c.dtype == torch.bfloat16

    def layers(self):
        if self.overlapping():
            if self.ws_gdn_layers is None:
                self.ws_gdn_layers = [torch.empty_like(self.ws_gdn) for _ in self.gdn]
                self.side = torch.cuda.Stream(self.dev)
            main = torch.cuda.current_stream(self.dev)
            # the side stream starts this round's state writes only after everything the main
            # stream did before (the previous commit read the last round's scratch)
            self.side.wait_stream(main)
        ia = ig = 0
        for kind in self.pattern:
            if kind == "attn":
                if self.overlapping():
                    main.wait_stream(self.side)  # the state writes run beside GDN layers only
                a = self.attn[ia]
                ia += 1
                if self.cfg.rope:
                    ddt.tree_attn_rope(a["q"], a["k_new"], a["v_new"], self.tree["depth"], self.cfg.rope[0],
                                       self.cfg.rope[1], a["k_cache"], a["v_cache"], self.prefix_len,
                                       self.tree["anc"], ws=self.ws_attn,
                                       out={"o": a["out"], "k_tree": a["k_tree"], "v_tree": a["v_tree"]})
                elif self.block_table is not None:
                    ddt.tree_attn_paged(a["q"], a["k_cache"], a["v_cache"], self.block_table, self.prefix_len,
                                        a["k_tree"], a["v_tree"], self.tree["anc"], ws=self.ws_attn, out=a["out"])
                else:
                    ddt.tree_attn(a["q"], a["k_cache"], a["v_cache"], self.prefix_len, a["k_tree"], a["v_tree"],
                                  self.tree["anc"], ws=self.ws_attn, out=a["out"])
            else:
                g = self.gdn[ig]
                if self.overlapping():
                    ws = self.ws_gdn_layers[ig]
                    ddt.gdn_tree_step_deferred(g["x"], g["conv_w"], g["conv_state"], g["v"], g["beta"], g["g"],
                                               g["S"], self.tree["parent"], self.cfg.L, ws, out=g["out"])
                    ev = torch.cuda.Event()
                    ev.record(main)
                    self.side.wait_event(ev)
                    ddt.gdn_tree_states(g["S"], g["out"]["S_scratch"], ws, stream=self.side)
                else:
                    ddt.gdn_tree_step(g["x"], g["conv_w"], g["conv_state"], g["v"], g["beta"], g["g"], g["S"],
                                      self.tree["parent"], self.cfg.L, ws=self.ws_gdn, out=g["out"],
                                      store_states=not self.cfg.replay)
                ig += 1

    def accept(self):
        if self.cfg.sampled:
            ddt.tree_accept_sampled(self.target_logits, self.gumbel, self.temperature, self.tree["tok"],
                                    self.tree["parent"], self.cfg.L, ws=self.ws_acc, out=self.acc)
        else:
            ddt.tree_accept(self.target_logits, self.tree["tok"], self.tree["parent"], self.cfg.L,
                            ws=self.ws_acc, out=self.acc)

    def commit(self):
        if self.overlapping() and self.side is not None:
            torch.cuda.current_stream(self.dev).wait_stream(self.side)  # every state written
        kv = [(a["k_tree"], a["v_tree"], a["k_cache"], a["v_cache"]) for a in self.attn]
        if self.cfg.replay:
            # KV rows are copied; the recurrent state is advanced along the accepted path
            # after the commit has marked the sequences that may not be written
            ddt.commit(self.acc["acc_rows"], self.acc["acc_len"], self.prefix_len, kv, (), B=self.cfg.B,
                       block_table=self.block_table)
            ddt.gdn_replay(self.acc["acc_rows"], self.acc["acc_len"],
                           [(g["x"], g["conv_w"], g["v"], g["beta"], g["g"], g["S"], g["conv_state"])
                            for g in self.gdn], B=self.cfg.B)
        else:
            ddt.commit(self.acc["acc_rows"], self.acc["acc_len"], self.prefix_len, kv,
                       [(g["out"]["S_scratch"], g["S"], g["out"]["conv_scratch"], g["conv_state"])
                        for g in self.gdn], B=self.cfg.B, block_table=self.block_table)
        # the bonus token of this round is the root of the next one; a sequence that was
        # not committed (acc_len -1: malformed walk, capacity or bad rows) keeps its root,
        # so no token drops out of its sequence
        self.root_token.copy_(torch.where(self.acc["acc_len"] >= 0, self.acc["bonus"], self.root_token))

    def __call__(self):
        self.build()
        self.layers()
        self.accept()
        self.commit()

    # ------------------------------------------------------------ seeded synthetic inputs
    def fill_random(self, seed=0, draft_sigma=3.0, plant_p=0.6, target_sigma=3.0, target_plant=0.7):
        """Seeded device-side draws with the workload's distributions; the target
        plant uses the tree of the current drafter logits (built once here)."""
        c, dev = self.cfg, self.dev
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        rn = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32)
        ru = lambda *s: torch.rand(*s, generator=gen, device=dev, dtype=torch.float32)
        z = draft_sigma * rn(c.n, c.L, c.V)
        hit = ru(c.n, c.L) < plant_p
        where = torch.randint(0, c.V, (c.n, c.L), generator=gen, device=dev)
        zmax = z.amax(dim=-1)
        zi = z.view(-1, c.V)
        rows = torch.nonzero(hit.view(-1)).flatten()
        zi[rows, where.view(-1)[rows]] = zmax.view(-1)[rows] + 8.0
        self.draft_logits.copy_(z)
        del z, zi
        for a in self.attn:
            for k in ("q", "k_new", "v_new", "k_cache", "v_cache") if c.rope else \
                    ("q", "k_tree", "v_tree", "k_cache", "v_cache"):
                a[k].copy_(rn(*a[k].shape))
        for g in self.gdn:
            g["x"].copy_(rn(*g["x"].shape))
            g["v"].copy_(rn(*g["v"].shape))
            g["beta"].copy_(ru(*g["beta"].shape))
            g["g"].copy_(0.9 + 0.1 * ru(*g["g"].shape))
            g["S"].copy_(rn(*g["S"].shape) / c.dk ** 0.5)
            g["conv_state"].copy_(rn(*g["conv_state"].shape))
            g["conv_w"].copy_((2 * ru(*g["conv_w"].shape) - 1) / c.W ** 0.5)
        # target: N(0, sigma); rows at depth d get the drafter's top-1 of depth d+1 as argmax w.p. target_plant
        self.build()
        depth = self.tree["depth"].long()
        top1 = self.draft_logits.float().argmax(dim=-1)               # [n][L]
        y = target_sigma * rn(c.n, c.T, c.V)
        thit = ru(c.n, c.L) < target_plant
        for s in range(c.n):
            for d in range(c.L):
                if not bool(thit[s, d]):
                    continue
                rows_d = torch.nonzero(depth[s] == d).flatten()
                if rows_d.numel():
                    y[s, rows_d, top1[s, d]] = y[s, rows_d].amax(dim=-1) + 1.0
        self.target_logits.copy_(y)
        del y
        if c.sampled:
            u = ru(c.n, c.T, c.V).clamp_(1e-12, 1.0 - 1e-7)
            self.gumbel.copy_(-torch.log(-torch.log(u)))
            del u
        torch.cuda.synchronize(dev)
