"""Host-side model of the GEMV kernel's weight addressing (launch plan, task
split, cursors, clamping), used to prove on the CPU that every load of every
lane of every wave stays inside the weight buffer for a given call shape.

It restates, in Python, the integer arithmetic of plan() in q4_host.h and of
the cursor / load() code of gemv_kernel in q4_kernels.h; keep the two in step
(test_addressing.py runs it over the parity-test shapes and edge cases)."""
Q4K_BYTES = 144
Q40_PAIR = 36
U32 = 0xFFFFFFFF


def row_bytes(fmt, K):
    """ceil(K/256) super-blocks (Q4_K rows may end inside the last one),
    K/32 blocks (Q4_0)."""
    return (K + 255) // 256 * 144 if fmt == "q4k" else (K // 32) * 18


def mpadk(K):
    """Columns the batched kernel stages: whole 256-column steps."""
    return (K + 255) // 256 * 256


def pow2ceil(v):
    p = 1
    while p < v:
        p <<= 1
    return p


def plan(M, K, rows, RR, moe, npairs_max, cus=256, bpc=None, wpb=None, lg=None):
    # single-token calls with rows of at most 64 units run 256-thread
    # workgroups (4 waves), longer single-token rows and dense batched calls
    # 512-thread ones (8 waves), up to 2 per CU; expert calls 256-thread ones
    # at M = 2..4 (3 per CU) and 768-thread ones otherwise (1 per CU)
    moe4 = moe and 2 <= M <= 4
    if wpb is None:
        wpb = (4 if moe4 else 12) if moe else (4 if M == 1 and (K + 63) // 64 <= 64 else 8)
    upr = (K + 63) // 64
    xr = not moe and M == 1 and upr <= 64
    if bpc is None:
        # (register-resident single-token calls: up to 3 per CU)
        bpc = (3 if moe4 else 1) if moe else (3 if xr else 2)
    if lg is None:
        lg = 64 if upr >= 64 else max(4, pow2ceil(upr))
        if M <= 2 and upr > 64 and not moe:
            need32 = ((rows + 2 * RR - 1) // (2 * RR) + wpb - 1) // wpb
            if need32 % cus == 0 or need32 >= 2 * cus:
                lg = 32  # long dense rows at one or two tokens, filling the CUs evenly
        if moe and 2 <= M <= 4 and lg >= 32:
            lg //= 2  # expert calls of 2-4 tokens: two units per lane and row
    upl = (upr + lg - 1) // lg
    rgw = 64 // lg
    nrg = (rows + RR - 1) // RR
    if moe:
        nrg = (nrg + rgw - 1) // rgw * rgw
        ntasks = 0
        tasks = npairs_max * (nrg // rgw)
    else:
        ntasks = (nrg + rgw - 1) // rgw
        tasks = ntasks
    blocks = min(cus * bpc, (tasks + wpb - 1) // wpb)
    # at least two steps per wave, down to one workgroup per CU
    blocks = min(blocks, max(cus, (tasks * upl // 2 + wpb - 1) // wpb))
    blocks = max(1, blocks)
    return dict(upr=upr, lg=lg, upl=upl, rgw=rgw, nrg=nrg, ntasks=ntasks, nwaves=blocks * wpb)


def unit_off(fmt, u):
    return (u >> 2) * Q4K_BYTES if fmt == "q4k" else (u * 32 if fmt == "q4_0s" else u * Q40_PAIR)


def loads(fmt, M, N, K, RR, nmat, moe_experts=None, E=1, **kw):
    """Yield (matrix, byte offset, nbytes) of every load (a superset: each
    visited cursor in its normal and its idle form); moe_experts is the list
    of unique valid experts the in-kernel dedupe would produce."""
    moe = moe_experts is not None
    pl = plan(M, K, N, RR, moe, kw.get("npairs_max", 1), **{k: v for k, v in kw.items()
                                                             if k in ("cus", "bpc", "wpb", "lg")})
    rb = row_bytes(fmt, K)
    upr, lg, upl, rgw = pl["upr"], pl["lg"], pl["upl"], pl["rgw"]
    u_last = upr - 1
    if moe:
        tpe = pl["nrg"] // rgw
        nu = len(moe_experts)
        ntasks = nu * tpe
    else:
        tpe = 1
        ntasks = pl["ntasks"]
    for gw in range(pl["nwaves"]):
        t0, t1, ts = gw, ntasks, pl["nwaves"]
        # cursors visited: the first one always, then every task < t1
        curs = []
        ue = t0 // tpe if moe else 0
        rgt = t0 - ue * tpe if moe else t0
        t, ui = t0, 0
        curs.append((t, ui, ue, rgt))
        while True:
            ui += 1
            if ui == upl:
                ui = 0
                t += ts
                rgt += ts
                if moe and rgt >= tpe:
                    ue += rgt // tpe
                    rgt -= (rgt // tpe) * tpe
            if t >= t1:
                break
            curs.append((t, ui, ue, rgt))
        for (t, ui, ue, rgt) in curs:
            for lane in range(64):
                gi, li = lane // lg, lane % lg
                u = li + ui * lg
                in_row = u <= u_last
                uoff = unit_off(fmt, li) + ui * unit_off(fmt, lg) if in_row else unit_off(fmt, u_last)
                g = (li & 3) if in_row else (u_last & 3)
                qoff = uoff + 16 + 32 * g if fmt == "q4k" else uoff
                R0 = rgt * rgw * RR
                ubase = moe_experts[min(ue, nu - 1)] * N if (moe and nu > 0) else 0
                R0c = max(0, min(R0, N - 1))
                lrow_max = N - 1 - R0c
                for r in range(RR):
                    # the lane part is 32-bit unsigned arithmetic in the kernel
                    lr = min(gi * RR + r + (R0 - R0c), lrow_max) & U32
                    ro = (lr * rb) & U32
                    sbase = (ubase + R0c) * rb
                    if fmt == "q4_0s":
                        # split arrays: nibble blocks 2u and min(2u+1, nb-1)
                        # (offsets into the quants), and their f16 scales
                        # (yielded as matrix 1: offsets into the scales)
                        nb = K // 32
                        uu = u if in_row else u_last
                        for blk in (2 * uu, min(2 * uu + 1, nb - 1)):
                            qo = (ubase + R0c) * nb * 16 + ((lr * nb * 16 + 16 * blk) & U32)
                            so = (ubase + R0c) * nb * 2 + ((lr * nb * 2 + 2 * blk) & U32)
                            yield 0, qo, 16
                            yield 1, so, 2
                        continue
                    for mt in range(nmat):
                        if fmt == "q4k":
                            yield mt, sbase + ((ro + uoff) & U32), 16
                            yield mt, sbase + ((ro + qoff) & U32), 16
                            yield mt, sbase + ((ro + qoff) & U32) + 16, 16
                        else:
                            yield mt, sbase + ((ro + uoff) & U32), 16
                            yield mt, sbase + ((ro + uoff) & U32) + 16, 16
                            yield mt, sbase + ((ro + uoff) & U32) + 32, 4
                        # idle form of the same cursor (loads past the wave's
                        # last step): every lane reads the task's first bytes
                        yield mt, sbase, 16
                        yield mt, sbase + 16, 16
                        yield mt, sbase + 32, 16 if fmt == "q4k" else 4


def check(fmt, M, N, K, RR, nmat, moe_experts=None, E=1, **kw):
    rows_total = (E if moe_experts is not None else 1) * N
    if fmt == "q4_0s":
        limits = [rows_total * (K // 32) * 16, rows_total * (K // 32) * 2]
        aligns = [16, 2]
    else:
        rb = row_bytes(fmt, K)
        limits, aligns = [rows_total * rb] * 2, [4, 4]
    n = 0
    for mt, off, nb in loads(fmt, M, N, K, RR, nmat, moe_experts, E, **kw):
        limit = limits[mt] if fmt == "q4_0s" else limits[0]
        assert 0 <= off and off + nb <= limit, (fmt, M, N, K, mt, off, nb, limit)
        a = aligns[mt] if fmt == "q4_0s" else 4
        assert off % a == 0, ("word loads need %d-byte alignment" % a, fmt, K, off)
        n += 1
    return n


# ---------------------------------------------------------------------------
# Matrix-core kernel (batched calls, M >= 2): q4_mfma.h and run_mfma_m().
# ---------------------------------------------------------------------------
LDS_CAP = 160 * 1024 - 1024  # dynamic LDS the batched kernel may ask for
Q40_WAVE_BYTES = 16 * 144    # Q4_0 tile-step copy per wave


def sums_stride(M):
    return M + (M & 1)


def mlayout(fmt, M, K, pure=False):
    """Byte offsets of the kernel's LDS regions (mlayout() in q4_mfma.h)."""
    K = mpadk(K)
    aux = 0 if pure else (K // 8 + 1) * 2 * M * 16
    aux_bytes = 0 if pure else ((K // 256) * 4 * 2 * M * 4 if fmt == "q4k"
                                else (K // 32) * sums_stride(M) * 4)
    exps = aux + aux_bytes
    part = exps + 64
    wbuf = part + 2 * 8 * 64 * 8
    nbytes = wbuf + (8 * Q40_WAVE_BYTES if fmt != "q4k" else 0)
    return dict(frag=0, aux=aux, exps=exps, part=part, wbuf=wbuf, bytes=nbytes)


def mfma_ks(ntiles, steps, cus, waves_per_cu=8):
    """Waves per tile (mfma_ks() in q4_host.h)."""
    ks = 1
    while ks < 8 and 2 * ks <= steps and 4 * ntiles * ks < 3 * cus * waves_per_cu:
        ks *= 2
    return ks


def mfma_plan(fmt, M, K, N, nmat, cus=256, nexperts=1, pair=False):
    """pair: the SiLU-gated gate+up call, whose tiles are 8 gate rows and the
    same 8 up rows; its K split still comes from the 16-row tile count."""
    lds = mlayout(fmt, M, K)["bytes"]
    wgc = max(1, min(2, LDS_CAP // lds))
    ntiles = nmat * nexperts * ((N + 15) // 16)
    steps = (K + 255) // 256
    KS = mfma_ks(ntiles, steps, cus)
    TG = 8 // KS
    if pair:
        ntiles = nexperts * ((N + 7) // 8)
    blocks = min(cus * wgc, (ntiles + TG - 1) // TG)
    return dict(lds=lds, blocks=blocks, ntiles=ntiles, TG=TG, KS=KS, steps=steps)


def mfma_positions(S, KS, nrounds, wave, PD):
    """(round, step) of every weight load a wave issues: the ring's first PD
    steps, then one load PD steps ahead for every slot the loop visits."""
    sl = wave % KS
    st0, st1 = sl * S // KS, (sl + 1) * S // KS
    ns = st1 - st0
    assert ns >= 1
    n = nrounds * ns
    visits = -(-n // PD) * PD
    return [(q // ns, st0 + q % ns) for q in range(visits + PD)]


def mfma_loads(fmt, M, N, K, nmat, cus=256, experts=None, umax=1, pair=False):
    """Yield (matrix, byte offset, nbytes) of every weight load; for the
    expert call, `experts` is the dedupe result and umax the host's bound on
    its length (which sizes the grid and the K split)."""
    pl = mfma_plan(fmt, M, K, N, nmat, cus, umax if experts is not None else 1, pair)
    rb = row_bytes(fmt, K)
    SB, PD = 144, (2 if fmt == "q4k" else 3)
    S, KS = pl["steps"], pl["KS"]
    while KS > S:  # the kernel's own clamp
        KS //= 2
    shift = 3 if pair else 4
    tpm = (N + (1 << shift) - 1) >> shift
    nu = len(experts) if experts is not None else 1
    per_mat = nu * tpm
    ntiles = (1 if pair else nmat) * per_mat
    if ntiles == 0:
        return
    TG, G = 8 // KS, pl["blocks"]
    nrounds = (ntiles + G * TG - 1) // (G * TG)
    for b in range(G):
        for wave in range(8):
            grp = wave // KS
            for (r, st) in mfma_positions(S, KS, nrounds, wave, PD):
                rr = min(r, nrounds - 1)
                traw = (rr * G + b) * TG + grp
                idle = r >= nrounds or traw >= ntiles
                t = min(traw, ntiles - 1)
                tmt = 1 if (nmat == 2 and not pair and t >= per_mat) else 0
                rem = t - tmt * per_mat
                u = rem // tpm if experts is not None else 0
                row0 = (rem - u * tpm) << shift
                ebase = experts[u] * N if experts is not None else 0
                base = (ebase + row0) * rb
                for lane in range(64):
                    jrow, c = lane & 15, lane >> 4
                    mt = (1 if jrow >= 8 else 0) if pair else tmt
                    lr = min(jrow & 7 if pair else jrow, N - 1 - row0) & U32
                    off = 0 if idle else (lr * rb + st * SB) & U32
                    if fmt == "q4k":
                        co = 0 if idle else 16 * c
                        yield mt, base + off, 16
                        yield mt, base + off + co + 16, 16
                        yield mt, base + off + co + 80, 16
                    elif fmt == "q4_0s":
                        # split arrays: nibble chunks lane, lane + 64 (row ch // 8,
                        # block ch % 8, clamped to the row's last block) as
                        # matrix 0, their f16 scales as matrix 1
                        nb = K // 32
                        for k in range(2):
                            ch = lane + 64 * k
                            ro = min(ch >> 3, N - 1 - row0)
                            gb = min(st * 8 + (ch & 7), nb - 1)
                            qo = 0 if idle else (ro * nb * 16 + 16 * gb) & U32
                            so = 0 if idle else (ro * nb * 2 + 2 * gb) & U32
                            yield 0, (ebase + row0) * nb * 16 + qo, 16
                            yield 1, (ebase + row0) * nb * 2 + so, 2
                    else:
                        # a partial last step clamps its chunk columns to
                        # the row's last 16 bytes
                        last_col = 18 * (K // 32 - 8 * (S - 1)) - 16
                        for k in range(3):
                            ch = min(lane + 64 * k, 143)
                            ro = (min(ch // 9, N - 1 - row0) * rb) & U32
                            col = (ch % 9) * 16
                            if st == S - 1:
                                col = min(col, last_col)
                            o = 0 if idle else (ro + st * SB + col) & U32
                            yield mt, base + o, 16


def mfma_check(fmt, M, N, K, nmat, cus=256, experts=None, umax=1, E=1, pair=False):
    pl = mfma_plan(fmt, M, K, N, nmat, cus, pair=pair)
    assert pl["lds"] <= LDS_CAP or M * K > 32768, (fmt, M, K, pl["lds"])
    rows = (E if experts is not None else 1) * N
    if fmt == "q4_0s":
        limits, aligns = [rows * (K // 32) * 16, rows * (K // 32) * 2], [16, 2]
    else:
        limits, aligns = [rows * row_bytes(fmt, K)] * 2, [4, 4]
    n = 0
    for mt, off, nb in mfma_loads(fmt, M, N, K, nmat, cus, experts, umax, pair):
        lim = limits[mt] if fmt == "q4_0s" else limits[0]
        assert 0 <= off and off + nb <= lim, (fmt, M, N, K, mt, off, nb, lim)
        a = aligns[mt] if fmt == "q4_0s" else 4
        assert off % a == 0, ("loads need %d-byte alignment" % a, fmt, K, off)
        n += 1
    return n


def mfma_lds_check(fmt, M, K0):
    """Every LDS byte the kernel writes while staging or reads while
    computing lies inside its region, and every fragment and sum a compute
    step reads was written by the staging."""
    ly = mlayout(fmt, M, K0)
    K = mpadk(K0)  # staged columns: real pieces, then zero pieces up to K
    ppt = K // 8
    frag_w, aux_w = set(), set()
    for m in range(M):
        for pp in range(ppt):
            for h in range(2):
                o = ((2 * m + h) * (K // 8 + 1) + pp) * 16
                assert ly["frag"] <= o and o + 16 <= ly["aux"]
                frag_w.add(o)
            if pp & 3 == 0:
                g32 = pp >> 2
                if fmt == "q4_0":
                    o = ly["aux"] + (g32 * sums_stride(M) + m) * 4
                    assert o + 4 <= ly["exps"]
                    aux_w.add(o)
                else:
                    sb, J = g32 >> 3, g32 & 7
                    half = ((sb * 4 + (J >> 1)) * 2 * M + 2 * m) * 2 + (J & 1)
                    for hh in (half, half + 2):
                        o = ly["aux"] + 2 * hh
                        assert o + 2 <= ly["exps"]
                        aux_w.add(o)
    S = K // 256
    for st in range(S):
        for lane in range(64):
            jrow, c = lane & 15, lane >> 4
            i = min(jrow, 2 * M - 1)
            if fmt == "q4k":
                pb = st * 32 + 8 * (c >> 1) + 2 * (c & 1)
                pps = [pb + 16 * h + s + 4 * n for h in range(2) for s in range(2)
                       for n in range(2)]
                o = ly["aux"] + ((st * 4 + c) * 2 * M + i) * 4
                assert o + 4 <= ly["exps"]
                assert o in aux_w and o + 2 in aux_w
            else:
                pps = []
                MP = sums_stride(M)
                for k in range(4):
                    blk = st * 8 + 2 * k
                    pps += [blk * 4 + c, blk * 4 + 4 + c]
                    for bb in (blk, blk + 1):
                        o = ly["aux"] + (bb * MP + min(2 * c, MP - 2)) * 4
                        assert o + 8 <= ly["exps"]
                        # token 2c (and 2c + 1) sums exist when those tokens do
                        for hm in range(2):
                            if 2 * c + hm < M:
                                assert o + 4 * hm in aux_w
                    # the wave's tile-step copy: words read by this lane
                    h = c & 1
                    for wd in [jrow * 36 + 9 * k + 2 * h + d for d in (0, 1, 2, 5, 6)] + \
                              [jrow * 36 + 9 * k + 4 - 4 * h]:
                        assert 0 <= wd * 4 and wd * 4 + 4 <= Q40_WAVE_BYTES
            for pp in pps:
                o = (i * (K // 8 + 1) + pp) * 16
                assert o + 16 <= ly["aux"] and o in frag_w
    if fmt == "q4_0":
        for lane in range(64):
            for k in range(3):
                ch = min(lane + 64 * k, 143)
                assert ch * 16 + 16 <= Q40_WAVE_BYTES
    assert ly["part"] + 2 * 8 * 64 * 8 == ly["wbuf"]
    return True


# ---------------------------------------------------------------------------
# Router (q4_router.h): one workgroup of 8 waves per token.
# ---------------------------------------------------------------------------
def router_loads(E, K, waves=8, rows=4):
    """Yield (byte offset, nbytes) of every weight load of one token's
    workgroup (router_kernel's logits loop)."""
    upr = K // 64
    lgw = 4
    while lgw < upr and lgw < 64:
        lgw <<= 1
    rpp = 64 // lgw
    upl = (upr + lgw - 1) // lgw
    rb = (K // 32) * 18
    step = waves * rpp * rows
    for wave in range(waves):
        e0 = wave * rpp * rows
        while e0 < E:
            for lane in range(64):
                gi, li = lane // lgw, lane % lgw
                for i in range(upl):
                    u = li + lgw * i
                    uc = u if u < upr else upr - 1
                    for q in range(rows):
                        e = min(e0 + q * rpp + gi, E - 1)
                        base = e * rb + uc * Q40_PAIR
                        yield base, 16
                        yield base + 16, 16
                        yield base + 32, 4
            e0 += step


def router_check(E, K):
    limit = E * (K // 32) * 18
    n = 0
    for off, nb in router_loads(E, K):
        assert 0 <= off and off + nb <= limit, (E, K, off, nb, limit)
        n += 1
    return n


# ---------------------------------------------------------------------------
# Expert down-projection (q4_moe_down.h, run_down_m() in q4_host.h): one
# contiguous slice of the (unique expert, row group) space per workgroup of
# 4 waves.
# ---------------------------------------------------------------------------
def choose_lg_waste(upr):
    best, best_idle, best_slots = 4, 1 << 30, 1
    lg = 64
    while lg >= 4:
        slots = (upr + lg - 1) // lg * lg
        idle = slots - upr
        if 8 * idle <= slots:
            return lg
        if idle * best_slots < best_idle * slots:
            best, best_idle, best_slots = lg, idle, slots
        lg //= 2
    return best


def down_plan(N, K, npairs_max, cus=256, wgc=4, RR=1):
    upr = (K + 63) // 64
    lg = choose_lg_waste(upr)
    upl = (upr + lg - 1) // lg
    rgw = 64 // lg
    nrg = (N + RR - 1) // RR
    per_pass = 4 * rgw
    ks = (cus * wgc + npairs_max - 1) // npairs_max
    ks = max(1, min(ks, (nrg + per_pass - 1) // per_pass))
    return dict(upr=upr, lg=lg, upl=upl, rgw=rgw, nrg=nrg, per_pass=per_pass, ks=ks,
                blocks=ks * npairs_max)


def down_loads(N, K, experts, npairs_max, cus=256, wgc=4, RR=1):
    """Yield (byte offset, nbytes) of every weight load of the down kernel,
    for the dedupe result `experts` (unique valid ids): workgroup b serves
    expert b // ks and share b % ks of its row groups."""
    pl = down_plan(N, K, npairs_max, cus, wgc, RR)
    upr, lg, upl, rgw, nrg, per_pass, ks, G = (pl[k] for k in (
        "upr", "lg", "upl", "rgw", "nrg", "per_pass", "ks", "blocks"))
    rb = (K // 32) * 18
    for b in range(G):
        ux, part = divmod(b, ks)
        if ux >= len(experts):
            continue
        g0, g1 = part * nrg // ks, (part + 1) * nrg // ks
        if g0 >= g1:
            continue
        e = experts[ux]
        nsteps = -(-(g1 - g0) // per_pass) * upl
        for wave in range(4):
            for q in range(nsteps):
                pss, ui = divmod(q, upl)
                gw = min(g0 + pss * per_pass + wave * rgw, g1 - 1)
                R0 = gw * RR
                lrow_max = N - 1 - R0
                assert lrow_max >= 0
                for lane in range(64):
                    gi, li = lane // lg, lane % lg
                    uoff = min(li + ui * lg, upr - 1) * Q40_PAIR
                    for r in range(RR):
                        lr = min(gi * RR + r, lrow_max)
                        off = (e * N + R0) * rb + ((lr * rb + uoff) & U32)
                        yield off, 16
                        yield off + 16, 16
                        yield off + 32, 4


def down_check(N, K, experts, E, npairs_max, cus=256, wgc=4, RR=1):
    limit = E * N * (K // 32) * 18
    n = 0
    for off, nb in down_loads(N, K, experts, npairs_max, cus, wgc, RR):
        assert 0 <= off and off + nb <= limit, (N, K, off, nb, limit)
        assert off % 4 == 0
        n += 1
    return n


# ---------------------------------------------------------------------------
# K-sliced staging of the batched kernel (run_mfma_m() in q4_host.h,
# MSlice / mstage_slice in q4_mfma.h).
# ---------------------------------------------------------------------------
LDS_TOTAL = 160 * 1024


def mlayout_steps(fmt, M, steps, pure=False):
    K = steps * 256
    ntile = (M + 7) // 8
    aux = 0 if pure else (K // 8 + 1) * 2 * M * 16
    aux_bytes = 0 if pure else ((K // 256) * 4 * 2 * M * 4 if fmt == "q4k"
                                else (K // 32) * sums_stride(M) * 4)
    exps = aux + aux_bytes
    part = exps + 128
    wbuf = part + 2 * 8 * 64 * 8 * ntile
    return wbuf + (8 * Q40_WAVE_BYTES if fmt != "q4k" else 0)


def slice_plan(fmt, M, N, K, nmat=1, cus=256):
    """(whole, KS, npg, nsl, msl, budget) as run_mfma_m chooses them."""
    reserve = 2048 if M > 8 else 1024
    budget = LDS_TOTAL - reserve
    S = (K + 255) // 256
    ntiles = nmat * ((N + 15) // 16)
    ks = mfma_ks(ntiles, S, cus)
    whole = M * S * 256 <= 32768 and mlayout_steps(fmt, M, S) <= budget
    if whole:
        return True, ks, 1, 1, S, budget
    kse = ks
    while kse > S:
        kse //= 2
    lmax = -(-S // kse)
    nsl, msl, npg = 1, lmax, 1
    while mlayout_steps(fmt, M, -(-kse // npg) * msl) > budget:
        if msl > 1:
            nsl += 1
            msl = -(-lmax // nsl)
        else:
            assert npg < kse, "no slice fits"
            npg *= 2
    return False, kse, npg, nsl, msl, budget


def slice_ranges(S, KS, npg, nsl, sl, slice_):
    """(a, b, region) of wave position sl in a slice (MSlice::range)."""
    g, s = divmod(slice_, nsl)
    p0, p1 = g * KS // npg, (g + 1) * KS // npg
    if not p0 <= sl < p1:
        return 0, 0, 0
    s0 = sl * S // KS
    L = (sl + 1) * S // KS - s0
    return s0 + s * L // nsl, s0 + (s + 1) * L // nsl, sl - p0


def slice_check(fmt, M, N, K, nmat=1, cus=256):
    """Every wave position's steps are covered once, in order, across the
    slices; each sub-range fits its region of msl local steps, and regions
    stay inside the staged steps; the staged layout fits the LDS budget."""
    whole, KS, npg, nsl, msl, budget = slice_plan(fmt, M, N, K, nmat, cus)
    S = (K + 255) // 256
    if whole:
        assert mlayout_steps(fmt, M, S) <= budget
        return whole
    regions = -(-KS // npg)
    assert mlayout_steps(fmt, M, regions * msl) <= budget
    for sl in range(KS):
        seen = []
        for sc in range(npg * nsl):
            a, b, reg = slice_ranges(S, KS, npg, nsl, sl, sc)
            assert 0 <= b - a <= msl and reg < regions, (sl, sc, a, b, msl)
            seen += list(range(a, b))
        assert seen == list(range(sl * S // KS, (sl + 1) * S // KS)), (sl, seen)
    return whole


# ---------------------------------------------------------------------------
# Split-K batched GEMV (splitk_plan() in q4_host.h, the kStgSplitK path of
# q4_mfma.h): workgroup b serves tile group b // kp and K part b % kp.
# ---------------------------------------------------------------------------
SPLITK_ONE_STEPS = 4  # kSplitKOneSteps


def splitk_plan(fmt, M, N, K, cus=256):
    S = (K + 255) // 256
    ntiles = (N + 15) // 16
    ngroups = -(-ntiles // 8)
    kp = max(1, -(-cus // ngroups))
    kone = -(-S // SPLITK_ONE_STEPS)  # parts short enough for one-pass staging
    if kone <= 64 and kp < kone:
        kp = kone
    kp = min(S, kp)
    while True:
        msl = -(-S // kp)
        if mlayout_steps(fmt, 16, msl) <= LDS_TOTAL - 2048 or kp >= S:
            break
        kp += 1
    msl = -(-S // kp)
    return dict(kp=kp, msl=msl, ngroups=ngroups, S=S)


def splitk_role(b, T, kp, xcds=8):
    """(group, part) of split-K workgroup b of T (splitk_role() in q4_mfma.h):
    XCD b % 8 takes a contiguous run of the (group, part) pairs."""
    per, rem = divmod(T, xcds)
    x, i = b % xcds, b // xcds
    L = x * per + min(x, rem) + i
    return divmod(L, kp)


def splitk_check(fmt, M, N, K, cus=256):
    """Parts cover every step once; a part fits its staged steps and LDS;
    every partial and exponent index is inside its region; the plan does
    not depend on M."""
    pl = splitk_plan(fmt, M, N, K, cus)
    for M2 in (3, 8, 16):
        assert splitk_plan(fmt, M2, N, K, cus) == pl
    S, kp, msl, G = pl["S"], pl["kp"], pl["msl"], pl["ngroups"]
    assert mlayout_steps(fmt, M, msl) <= LDS_TOTAL - (2048 if M > 8 else 1024)
    steps = []
    PP = (M + 3) // 4  # part_pieces<M>()
    for q in range(kp):
        a, b, _ = slice_ranges(S, 1, 1, kp, 0, q)
        assert 1 <= b - a <= msl
        steps += list(range(a, b))
        if msl <= SPLITK_ONE_STEPS:
            # one-pass staging: the part's pieces fit PP per thread, and each
            # thread's (clamped) activation loads stay inside the row
            ppt = (b - a) * 32
            np_ = M * ppt
            assert np_ <= 512 * PP
            for tid in range(0, 512, 7):
                for k in range(PP):
                    pc = min(tid + 512 * k, np_ - 1)
                    m = pc // ppt
                    col = min(a * 256 + 8 * (pc - m * ppt), K - 8)
                    assert 0 <= m < M and 0 <= col and col + 8 <= K
    assert steps == list(range(S))
    roles = [splitk_role(b, G * kp, kp) for b in range(G * kp)]
    assert sorted(roles) == [divmod(L, kp) for L in range(G * kp)]  # a bijection
    for b in range(G * kp):
        g, q = roles[b]
        assert g < G
        for grp in range(8):
            t = g * 8 + grp
            for jrow in range(16):
                row = t * 16 + jrow
                if t < (N + 15) // 16 and row < N:
                    for m in range(M):
                        assert 0 <= (q * M + m) * N + row < kp * M * N
    return pl
